// prologue.hip -- the layer's prologue in front of the recurrence (gfx950):
// depthwise causal convolution with SiLU over the concatenated q, k, v
// channels, then per-head L2 normalization of q and k.
//
// "A Node-by-Node White-Box Walkthrough of a Quantized Hybrid Gated DeltaNet
// Language Model", Principais Contribuicoes: a token's path through a GDN
// sublayer runs through short convolutions before the gates and the
// recurrent scan.  The pages give no width; it is a parameter W (1..8):
//     y[t, c] = SiLU(bias[c] + sum_{j<W} w[c, j] * xe[t - (W-1) + j, c]),
// within each packed sequence, xe being the sequence's input extended on the
// left by its initial convolution state (the W-1 previous inputs, oldest
// first) or zeros; q, k <- y / sqrt(sum_head y^2 + eps) per (token, head);
// the final convolution state of each sequence is its last W-1 extended
// inputs, so a later call (a decode step) continues the convolution.
//
// Memory-bound (x read once, q/k/v written once).  Each lane owns 8
// consecutive channels (16 bytes of bf16) and walks a tile of kTile tokens,
// keeping the W-1 previous inputs of its channels in registers, so each
// input is read from memory once (plus a W-1 token halo per tile).  Inputs
// arrive in batches of kAhead tokens, double-buffered: the next batch is in
// flight while the current one is computed.  A head of d_k channels is
// d_k / 8 consecutive lanes; its sum of squares is a DPP group sum.  SiLU
// uses the hardware exponential and reciprocal.  A tile in which a sequence
// starts (once per sequence in a prefill, every token at decode) is walked
// token by token instead.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_seqmap.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 64;      // tokens per tile
constexpr int kAhead = 4;      // tokens per load batch (double-buffered)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One token's 8 channels as loaded (packed until used).
template <bool BF> struct Raw;
template <> struct Raw<true> { u32x4 a; };
template <> struct Raw<false> { f32x4 a, b; };

template <bool BF>
__device__ __forceinline__ Raw<BF> load_raw(const void* x, int64_t idx) {
  Raw<BF> r;
  if constexpr (BF) {
    r.a = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(x) + idx));
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(x) + idx);
    r.a = __builtin_nontemporal_load(p);
    r.b = __builtin_nontemporal_load(p + 1);
  }
  return r;
}

template <bool BF>
__device__ __forceinline__ void unpack(const Raw<BF>& r, float (&v)[8]) {
  if constexpr (BF) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(r.a[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(r.a[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = r.a[i];
      v[4 + i] = r.b[i];
    }
  }
}

__device__ __forceinline__ void store_y8(void* out, bool bf16, int64_t idx,
                                         const float (&v)[8]) {
  if (bf16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(
        w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + idx));
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p + 1);
  }
}

// Sum over the lph lanes of a head (lph in {2, 4, 8, 16}, uniform).
__device__ __forceinline__ float head_sum(float v, int lph) {
  switch (lph) {
    case 2: return group_sum<2>(v);
    case 4: return group_sum<4>(v);
    case 8: return group_sum<8>(v);
    default: return group_sum<16>(v);
  }
}

// Sequence containing token t (first n with cu[n+1] > t), or one sequence.
__device__ __forceinline__ int seq_of(const PrologueParams& p, int64_t t) {
  if (!p.cu) return 0;
  int lo = 0, hi = p.N - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (p.cu[mid + 1] > t) hi = mid; else lo = mid + 1;
  }
  return lo;
}
// Token range of sequence n, clamped into [0, T] (device offsets are not
// visible to the host checks).
__device__ __forceinline__ int64_t seq_beg(const PrologueParams& p, int n) {
  int64_t b, e;
  seq_bounds(p.cu, n, (int32_t)p.T, p.T, b, e);
  return b;
}
__device__ __forceinline__ int64_t seq_end(const PrologueParams& p, int n) {
  int64_t b, e;
  seq_bounds(p.cu, n, (int32_t)p.T, p.T, b, e);
  return e;
}

// One token of one lane: convolution over the carried inputs and x, SiLU,
// the head's L2 norm (q and k), the output store, and the carried inputs
// shifted by one.
template <int W>
struct LaneCtx {
  float w[8][W], bias[8];
  void* obase;
  int64_t ostride;
  bool active, norm, bf_out;
  int lph;
  float eps;
};

template <int W>
__device__ __forceinline__ void conv_token(const LaneCtx<W>& L,
                                           float (&ring)[W > 1 ? W - 1 : 1][8],
                                           const float (&xv)[8], int tu) {
  constexpr int R = W - 1;
  float y[8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = L.bias[i];
#pragma unroll
    for (int r = 0; r < R; ++r) acc += L.w[i][r] * ring[r][i];
    acc += L.w[i][R] * xv[i];
    y[i] = silu_fast(acc);
    ss += y[i] * y[i];
  }
#pragma unroll
  for (int r = 0; r + 1 < R; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) ring[r][i] = ring[r + 1][i];
  if constexpr (R > 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) ring[R - 1][i] = xv[i];
  }
  ss = head_sum(ss, L.lph);
  if (L.norm) {
    const float inv = rsqrtf(ss + L.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] *= inv;
  }
  if (L.active) store_y8(L.obase, L.bf_out, (int64_t)tu * L.ostride, y);
}

// The carried inputs at the start of sequence n: its initial state or zeros.
template <int W>
__device__ __forceinline__ void state_ring(const PrologueParams& p, int n,
                                           int64_t c0,
                                           float (&ring)[W > 1 ? W - 1 : 1][8]) {
  constexpr int R = W - 1;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ring[r][i] = p.s0 ? p.s0[((int64_t)n * p.C + c0 + i) * R + r] : 0.f;
}

template <int W>
__device__ __forceinline__ void store_state(const PrologueParams& p, int n,
                                            int64_t c0,
                                            const float (&ring)[W > 1 ? W - 1 : 1][8]) {
  constexpr int R = W - 1;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < 8; ++i) p.sF[((int64_t)n * p.C + c0 + i) * R + r] = ring[r][i];
}

template <int W, bool BF>
__global__ __launch_bounds__(kThreads) void prologue_kernel(PrologueParams p) {
  constexpr int R = W - 1;                  // inputs carried between tokens
  constexpr int kBatches = kTile / kAhead;
  const int64_t gidx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t groups = p.C / 8;
  const bool active = gidx < groups;
  const int64_t c0 = 8 * (active ? gidx : groups - 1);
  const int64_t cq = (int64_t)p.h_k * p.d_k;
  const bool is_q = c0 < cq, is_k = !is_q && c0 < 2 * cq;

  const int64_t t0 = (int64_t)blockIdx.y * kTile;
  const int64_t t1 = min(t0 + (int64_t)kTile, p.T);
  const int last = (int)(t1 - t0) - 1;        // last token of the tile
  // This lane's channels at the tile's first token; tokens are C apart.
  const void* xt0 = BF ? (const void*)(static_cast<const uint16_t*>(p.x) + t0 * p.C + c0)
                       : (const void*)(static_cast<const float*>(p.x) + t0 * p.C + c0);
  const int C32 = (int)p.C;
  // First batch of inputs, issued before anything else.
  Raw<BF> cur[kAhead], nxt[kAhead];
#pragma unroll
  for (int u = 0; u < kAhead; ++u) cur[u] = load_raw<BF>(xt0, min(u, last) * C32);

  LaneCtx<W> L;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int j = 0; j < W; ++j) L.w[i][j] = p.w[(c0 + i) * W + j];
    L.bias[i] = p.bias ? p.bias[c0 + i] : 0.f;
  }
  const int64_t cv = p.C - 2 * cq;
  L.ostride = is_q || is_k ? cq : cv;
  const int64_t ooff = t0 * L.ostride + (is_q ? c0 : is_k ? c0 - cq : c0 - 2 * cq);
  L.bf_out = p.out_bf16 != 0;
  L.obase = L.bf_out ? (void*)(static_cast<uint16_t*>(is_q ? p.q : is_k ? p.k : p.v) + ooff)
                     : (void*)(static_cast<float*>(is_q ? p.q : is_k ? p.k : p.v) + ooff);
  L.active = active;
  L.norm = is_q || is_k;
  L.lph = p.d_k / 8;
  L.eps = p.eps;

  int n = seq_of(p, t0);
  const int64_t beg = seq_beg(p, n), end = seq_end(p, n);
  // Inputs of positions t0 - R .. t0 - 1: from x inside the sequence, else
  // from the sequence's initial state (or zeros).
  float ring[R > 0 ? R : 1][8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t pos = t0 - R + r;
    if (pos >= beg) {
      unpack<BF>(load_raw<BF>(xt0, (int)(pos - t0) * C32), ring[r]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        ring[r][i] = p.s0 ? p.s0[((int64_t)n * p.C + c0 + i) * R +
                                 max(pos - beg + R, (int64_t)0)] : 0.f;
    }
  }
  if (end < t1) {
    // A sequence starts inside this tile (once per sequence in a prefill;
    // every token at decode): token by token, without prefetch, so that
    // the streaming loop below carries no second sequence's state.
    int64_t e = end;
    for (int tu = 0; tu <= last; ++tu) {
      const int64_t t = t0 + tu;
      if (t >= e && n < p.N - 1) {
        do {
          ++n;
          e = seq_end(p, n);
        } while (e <= t && n < p.N - 1);
        state_ring<W>(p, n, c0, ring);
      }
      float xv[8];
      unpack<BF>(load_raw<BF>(xt0, tu * C32), xv);
      conv_token<W>(L, ring, xv, tu);
      if (p.sF && L.active && t == e - 1) store_state<W>(p, n, c0, ring);
    }
    return;
  }

  // One sequence covers the whole tile: the token loop holds no load but
  // the double-buffered inputs.
#pragma unroll
  for (int bb = 0; bb < kBatches; ++bb) {
    if (bb + 1 < kBatches) {          // next batch in flight while this one runs
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        nxt[u] = load_raw<BF>(xt0, min(bb * kAhead + kAhead + u, last) * C32);
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int tu = bb * kAhead + u;
      if (tu <= last) {
        float xv[8];
        unpack<BF>(cur[u], xv);
        conv_token<W>(L, ring, xv, tu);
      }
    }
    if (bb + 1 < kBatches) {
#pragma unroll
      for (int u = 0; u < kAhead; ++u) cur[u] = nxt[u];
    }
  }
  // Final state of the sequence when it ends with the tile.
  if (p.sF && active && end == t1) store_state<W>(p, n, c0, ring);
}

// Final states of empty sequences: their initial state (or zeros).
__global__ __launch_bounds__(256) void empty_seq_state_kernel(PrologueParams p) {
  const int64_t per = (int64_t)p.C * (p.W - 1);
  const int64_t total = (int64_t)p.N * per;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int n = (int)(e / per);
    if (seq_end(p, n) == seq_beg(p, n)) p.sF[e] = p.s0 ? p.s0[e] : 0.f;
  }
}

template <int W>
hipError_t launch_w(const PrologueParams& p, hipStream_t stream) {
  const int64_t groups = p.C / 8;
  const dim3 grid((unsigned)((groups + kThreads - 1) / kThreads),
                  (unsigned)((p.T + kTile - 1) / kTile));
  if (p.io_bf16)
    hipLaunchKernelGGL((prologue_kernel<W, true>), grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((prologue_kernel<W, false>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prologue(const PrologueParams& p, hipStream_t stream) {
  if (p.sF && p.N > 0 && p.W > 1) {
    const int64_t total = (int64_t)p.N * p.C * (p.W - 1);
    const int64_t blocks = min((total + 255) / 256, (int64_t)1024);
    hipLaunchKernelGGL(empty_seq_state_kernel, dim3((unsigned)blocks), dim3(256),
                       0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.T == 0) return hipSuccess;
  switch (p.W) {
    case 1: return launch_w<1>(p, stream);
    case 2: return launch_w<2>(p, stream);
    case 3: return launch_w<3>(p, stream);
    case 4: return launch_w<4>(p, stream);
    case 5: return launch_w<5>(p, stream);
    case 6: return launch_w<6>(p, stream);
    case 7: return launch_w<7>(p, stream);
    case 8: return launch_w<8>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
