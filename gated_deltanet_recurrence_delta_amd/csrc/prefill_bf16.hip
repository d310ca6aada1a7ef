// prefill_bf16.hip -- chunked prefill of the gated delta rule on the bf16
// matrix cores of gfx950 (d_k = d_v = 128, chunk C = 64, bf16 q/k/v/z, fp32
// state).
//
// The rule ("Why Gated DeltaNet Survives 4-Bit Quantization", Abstract (iii))
//     S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
// is evaluated chunk by chunk in its WY / UT-transform form.  With S0 the
// state entering a chunk, ell = log a, G the chunk-local prefix sum of ell and
// E_ij = exp(G_i - G_j) on j <= i:
//     A = strict_lower(diag(b) (E o K K^T)),  T = (I + A)^{-1},
//     P = E o Q K^T (j <= i),
//     R = diag(b) (V - diag(e^G) K S0^T),     U = T R,
//     O = diag(e^G) Q S0^T + P U,
//     S = e^{G_L} S0 + K^T diag(e^{G_L - G}) U    (as S^T += K^T W).
// This equals the token-by-token rule in exact arithmetic.
//
// Four launches:
//  1. chunk_map: per-sequence chunk offsets (from cu_seqlens) and the
//     sequence of every chunk slot.
//  2. prep (one workgroup per chunk and value head, fully parallel): the
//     gates, the Grams K K^T and Q K^T, P and T = (I + A)^{-1} -- everything
//     that does not depend on the state.  T and P are written as hi/lo bf16
//     matrix-core fragments, and the chunk's K and Q, once per key head, as
//     the fragments the scan loads (one contiguous 1 KiB read per load).
//  3. scan (one workgroup per sequence, value head and 16-row slice of the
//     state): the state-dependent chain only, chunk after chunk, with the
//     16 x 128 fp32 state slice resident in the matrix-core accumulators.
//     Per chunk: K S0^T and Q S0^T (16 MFMAs/wave), R; T R; P U and the
//     state update -- three barriers.  The compute waves load their K / Q
//     fragments two chunks ahead; a fifth wave stages the other operands
//     two chunks ahead into LDS with direct-to-LDS loads.  With the tail
//     fused, the read-out goes to an fp32 staging buffer in the lanes' own
//     blocked order (one contiguous store per lane and chunk).
//  4. tail (with z; one workgroup per chunk and value head): the gated
//     RMSNorm of every token over the staged read-out, written head-major.
// Rows of S evolve independently, so slicing the state 8 ways gives 8x more
// workgroups than heads and fills the 256 compute units at batch 1.
//
// Precision.  q, k and v are exact bf16 inputs; every other operand of a
// product (S, R, U, W, T, P) is carried as a pair hi + lo of bf16 values
// (hi = rne(x), lo = rne(x - hi)): three MFMAs for a product of two such
// operands (hi.hi + hi.lo + lo.hi), two for a product with an exact input.
// Accumulation is fp32; the chunk-local decay prefix sum is formed in fp64.
//
// Matrix-core operand layout (v_mfma_f32_16x16x32_bf16): lane l, with
// g = l / 16 and c = l % 16, supplies A[c][8g .. 8g+7] and B[8g .. 8g+7][c]
// and receives D[4g .. 4g+3][c].  The 16x16x16 variant used inside the UT
// inverse takes A[c][4g .. 4g+3] and B[4g .. 4g+3][c].  Fragments written by
// prep are stored lane-major, so every fragment load in the scan is one
// contiguous 1 KiB read per wave.  bf16 tiles in LDS use an XOR swizzle of
// their 16-byte granules that keeps the 16 lanes of a read on distinct banks.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {

const bool kHaveBf16Mfma = true;

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kC = 64;        // chunk length
constexpr int kD = 128;       // d_k = d_v
constexpr int kThreads = 256;
// The scan splits each head's 128 state rows into slices of 16 rows; a
// slice is one workgroup whose compute wave w handles token tile w.
constexpr int kSliceRows = 16;
constexpr int kSlices = kD / kSliceRows;
constexpr int kLd = 68;       // fp32 row stride of the 64 x 64 work tiles
// Fragments of a 64 x 64 matrix used by T R and P U: (token tile w, k-step
// ks) for ks < (w < 2 ? 1 : 2) -> 6 fragments; each is 64 lanes x 16 bytes,
// stored hi then lo.  A chunk record holds T's then P's.
constexpr int kFrags = 6;
constexpr int kRecU4 = 2 * kFrags * 2 * 64;     // uint4 per chunk record
// K and Q of one chunk and key head as matrix-core fragments: fragment
// (token tile w, k-step ks) is 64 lanes x 16 bytes, lane (g, c) holding
// token 16 w + c, dims 32 ks + 8 g .. +7.  K's 16 fragments, then Q's.
constexpr int kKqU4 = 2 * 16 * 64;
__device__ __forceinline__ int frag_index(int w, int ks) {
  return w < 2 ? w : 2 * w - 2 + ks;
}

__device__ __forceinline__ int sw128(int r, int c) {
  return r * 128 + ((((c >> 3) ^ (r & 15)) << 3) | (c & 7));
}
__device__ __forceinline__ int sw64(int r, int c) {
  return r * 64 + ((((c >> 3) ^ ((r >> 1) & 7)) << 3) | (c & 7));
}

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma16(bf16x4_t a, bf16x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t ld8(const uint16_t* base, int off) {
  return *reinterpret_cast<const bf16x8_t*>(base + off);
}

__device__ __forceinline__ void split4(f32x4_t x, bf16x4_t& hi, bf16x4_t& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h = (__bf16)x[i];
    hi[i] = h;
    lo[i] = (__bf16)(x[i] - (float)h);
  }
}

__device__ __forceinline__ void store_split4(uint16_t* hi_arr, uint16_t* lo_arr,
                                             int off, f32x4_t x) {
  bf16x4_t h, l;
  split4(x, h, l);
  *reinterpret_cast<bf16x4_t*>(hi_arr + off) = h;
  *reinterpret_cast<bf16x4_t*>(lo_arr + off) = l;
}

// Barrier that orders LDS traffic only: global memory operations in flight
// (output stores) are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct Maps {
  int32_t* prefix;     // [N+1] first chunk slot of each sequence
  int32_t* chunk_seq;  // [QB] sequence of each chunk slot, -1 if unused
  uint4* rec;          // [QB][h_v][kRecU4] T and P fragments
  uint4* kqf;          // [QB][h_k][kKqU4] K and Q fragments
  float* gate;         // [QB][h_v][3][64]: e^G, e^{G_L - G}, b
  // Recurrent output for the tail pass, fp32, blocked as the scan's lanes
  // hold it: [QB][h_v][8 slices][4 token tiles][64 lanes] x 16 bytes, lane
  // (g, c) of tile w holding tokens 16 w + 4 g .. +3 of column 16 s + c.
  uint4* stage;
  int32_t QB;
};

__device__ __forceinline__ void seq_range(const PrefillParams& p, int n,
                                          int64_t& beg, int64_t& end) {
  if (p.cu) {
    beg = p.cu[n];
    end = p.cu[n + 1];
  } else {
    beg = (int64_t)n * p.seq_len;
    end = beg + p.seq_len;
  }
}

// ------------------------------------------------------------ chunk map --
__global__ __launch_bounds__(256) void chunk_map_kernel(PrefillParams p,
                                                        Maps m) {
  if (threadIdx.x == 0) {
    int32_t acc = 0;
    for (int n = 0; n < p.N; ++n) {
      int64_t b, e;
      seq_range(p, n, b, e);
      m.prefix[n] = acc;
      acc += (int32_t)((e - b + kC - 1) / kC);
    }
    m.prefix[p.N] = acc;
  }
  __syncthreads();
  const int32_t total = m.prefix[p.N];
  for (int q = threadIdx.x; q < m.QB; q += 256) {
    int32_t s = -1;
    if (q < total) {
      int lo = 0, hi = p.N - 1;  // last n with prefix[n] <= q
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (m.prefix[mid] <= q) lo = mid; else hi = mid - 1;
      }
      s = lo;
    }
    m.chunk_seq[q] = s;
  }
}

// ----------------------------------------------------------------- prep --
// One workgroup per (chunk, value head).  K and Q are staged in LDS for the
// Grams; the Gram tiles then wait in registers while the same LDS is reused
// for A and T in fp32.
struct PrepLds {
  union {
    struct {
      uint16_t Kr[kC * kD];   // K chunk [token][dim]
      uint16_t Qr[kC * kD];   // Q chunk [token][dim]
    } kq;
    struct {
      float A32[kC][kLd];     // A (strictly lower blocks)
      float T32[kC][kLd];     // T
    } at;
  } u;
  double G[kC];
  float b[kC];
};

// Gram tile (TI, TJ) computed transposed, X_TI K_TJ^T, so that lane (g, c)
// holds row i = 16 TI + c at columns j = 16 TJ + 4g .. 4g+3: four
// consecutive entries of a row of A or P.
__device__ __forceinline__ f32x4_t gram_t(const uint16_t* X, const uint16_t* K,
                                          int TI, int TJ, int g, int c) {
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    acc = mfma32(ld8(K, sw128(16 * TJ + c, 32 * ks + 8 * g)),
                 ld8(X, sw128(16 * TI + c, 32 * ks + 8 * g)), acc);
  return acc;
}

// A tile: A_ij = b_i E_ij (K K^T)_ij for j < i, into A32.
__device__ __forceinline__ void a_tile(PrepLds& sm, f32x4_t v, int TI, int TJ,
                                       int g, int c) {
  const int i = 16 * TI + c, j0 = 16 * TJ + 4 * g;
  const double Gi = sm.G[i];
  const float bi = sm.b[i];
  f32x4_t a;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float E = expf((float)(Gi - sm.G[j0 + jj]));
    a[jj] = (j0 + jj) < i ? bi * E * v[jj] : 0.f;
  }
  *reinterpret_cast<f32x4_t*>(&sm.u.at.A32[i][j0]) = a;
}

// P tile values: P_ij = E_ij (Q K^T)_ij for j <= i (row i = 16 TI + c,
// columns 16 TJ + 4 g .. +3 of the lane).
__device__ __forceinline__ f32x4_t p_vals(const PrepLds& sm, f32x4_t v, int TI,
                                          int TJ, int g, int c) {
  const int i = 16 * TI + c, j0 = 16 * TJ + 4 * g;
  const double Gi = sm.G[i];
  f32x4_t pv;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float E = expf((float)(Gi - sm.G[j0 + jj]));
    pv[jj] = (j0 + jj) <= i ? E * v[jj] : 0.f;
  }
  return pv;
}

// Two column tiles of a row block -- A (columns 32 ks .. +15) and B (the
// next 16), each lane (g, c) holding four consecutive columns 4 g .. +3 of
// row c -- to the 32-wide operand fragment, lane (g, c) holding columns
// 8 g .. +7 of row c.  With 16-lane rows A = [A0 A1 A2 A3] and B = [B0 B1 B2
// B3], the fragment's first four columns are [A0 A2 B0 B2] and its last
// four [A1 A3 B1 B3]: a 32-lane swap gives [A0 A1 B0 B1] / [A2 A3 B2 B3], a
// 16-lane swap then the two halves.
__device__ __forceinline__ uint4 tiles_to_frag(bf16x4_t a, bf16x4_t b) {
  const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
  const auto s0 = __builtin_amdgcn_permlane32_swap(ua.x, ub.x, false, false);
  const auto t0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(ua.y, ub.y, false, false);
  const auto t1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
  return make_uint4(t0[0], t1[0], t0[1], t1[1]);
}

// P fragment (TI, ks) from its column tiles 2 ks (a) and 2 ks + 1 (b), as
// hi / lo bf16 into the record: each store of the wave writes 1 KiB of
// whole lines.
__device__ __forceinline__ void p_frag(uint4* rec, f32x4_t a, f32x4_t b, int TI,
                                       int ks, int lane) {
  bf16x4_t ah, al, bh, bl;
  split4(a, ah, al);
  split4(b, bh, bl);
  const int f = frag_index(TI, ks);
  rec[((kFrags + f) * 2 + 0) * 64 + lane] = tiles_to_frag(ah, bh);
  rec[((kFrags + f) * 2 + 1) * 64 + lane] = tiles_to_frag(al, bl);
}

// 16x16 fp32 tile products on the 16x16x16 op with hi/lo operands.  X is an
// LDS tile (row stride kLd); Y an LDS tile or the accumulator registers of a
// previous product (its output layout D[4g+i][c] is the B-operand layout).
__device__ __forceinline__ f32x4_t mm16(bf16x4_t xh, bf16x4_t xl, f32x4_t y,
                                        f32x4_t acc) {
  bf16x4_t yh, yl;
  split4(y, yh, yl);
  acc = mfma16(xh, yh, acc);
  acc = mfma16(xh, yl, acc);
  acc = mfma16(xl, yh, acc);
  return acc;
}
__device__ __forceinline__ void a_operand16(const float* X, int g, int c,
                                            bf16x4_t& h, bf16x4_t& l) {
  const float4 v = *reinterpret_cast<const float4*>(X + c * kLd + 4 * g);
  split4(f32x4_t{v.x, v.y, v.z, v.w}, h, l);
}
__device__ __forceinline__ f32x4_t b_operand16(const float* Y, int g, int c) {
  f32x4_t y;
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = Y[(4 * g + j) * kLd + c];
  return y;
}
__device__ __forceinline__ f32x4_t mm16_ll(const float* X, const float* Y,
                                           f32x4_t acc, int g, int c) {
  bf16x4_t xh, xl;
  a_operand16(X, g, c, xh, xl);
  return mm16(xh, xl, b_operand16(Y, g, c), acc);
}
__device__ __forceinline__ f32x4_t mm16_lr(const float* X, f32x4_t y,
                                           f32x4_t acc, int g, int c) {
  bf16x4_t xh, xl;
  a_operand16(X, g, c, xh, xl);
  return mm16(xh, xl, y, acc);
}

// T = (I + A)^{-1}, diagonal 16x16 blocks: lane (d = g, col = c) solves
// column col of block d by forward substitution.
__device__ __forceinline__ void t_diag(PrepLds& sm, int g, int c) {
  float(*A32)[kLd] = sm.u.at.A32;
  float(*T32)[kLd] = sm.u.at.T32;
  const int d = g, col = c;
  float x[16], s[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    x[k] = (k == col ? 1.f : 0.f) - s[k];
#pragma unroll
    for (int i = k + 1; i < 16; ++i) s[i] += A32[16 * d + i][16 * d + k] * x[k];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) T32[16 * d + i][16 * d + col] = x[i];
}

// Column block E of T below the diagonal, top to bottom (one wave; no other
// wave touches column E):  T_{d,E} = -T_dd sum_{E <= k < d} A_{d,k} T_{k,E}.
// The column's blocks stay in registers (their output layout is the B
// operand layout) and go to T32 only at the end, so every LDS read of the
// chain can be issued up front.
template <int E>
__device__ __forceinline__ void t_column(PrepLds& sm, int g, int c) {
  float(*A32)[kLd] = sm.u.at.A32;
  float(*T32)[kLd] = sm.u.at.T32;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t tc[4];
  tc[E] = b_operand16(&T32[16 * E][16 * E], g, c);
#pragma unroll
  for (int d = E + 1; d < 4; ++d) {
    f32x4_t z = zero;
#pragma unroll
    for (int k = E; k < d; ++k) z = mm16_lr(&A32[16 * d][16 * k], tc[k], z, g, c);
    tc[d] = -mm16_lr(&T32[16 * d][16 * d], z, zero, g, c);
  }
#pragma unroll
  for (int d = E + 1; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) T32[16 * d + 4 * g + i][16 * E + c] = tc[d][i];
}

__global__ __launch_bounds__(kThreads, 4) void prep_kernel(PrefillParams p,
                                                        Maps m) {
  __shared__ PrepLds sm;
  // Work item = (chunk, value head).  Blocks are dealt to the 8 XCDs
  // round-robin; the remap gives consecutive items -- the value heads that
  // share a key head, for one chunk -- to one XCD, so their K and Q meet in
  // its L2.
  const int nb = gridDim.x;
  const int lid = (nb & 7) == 0 ? (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3)
                                : blockIdx.x;
  const int q = lid / p.h_v, h = lid - q * p.h_v;
  const int n = m.chunk_seq[q];
  if (n < 0) return;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int hk = h / p.group;
  int64_t s_beg, s_end;
  seq_range(p, n, s_beg, s_end);
  const int64_t t0 = s_beg + (int64_t)(q - m.prefix[n]) * kC;
  const int L = (int)((s_end - t0) < kC ? (s_end - t0) : kC);
  const bool direct = p.direct != 0;
  uint4* rec = m.rec + ((int64_t)q * p.h_v + h) * kRecU4;

  // Wave 0 fetches the chunk's gate inputs first, so that waiting for them
  // (vector loads complete in order) does not wait for K and Q.
  float graw = 0.f, braw = 0.f;
  if (w == 0 && lane < L) {
    const int64_t gi = (t0 + lane) * p.h_v + h;
    graw = p.g[gi];
    braw = p.beta[gi];
  }
  // K (threads 0-127) and Q (128-255): 8 tokens x 16 bytes per thread, all
  // loads issued before any use.  Rows past the end of a short chunk repeat
  // its last token: they meet b = 0 in A, and P's rows there are never used.
  const int tb = (t & 127) >> 4, gr = t & 15;
  const uint16_t* src = static_cast<const uint16_t*>(t < 128 ? p.k : p.q);
  u32x4_t kv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int tok = min(8 * tb + j, L - 1);
    kv[j] = *reinterpret_cast<const u32x4_t*>(src + ((t0 + tok) * p.h_k + hk) * kD +
                                              8 * gr);
  }
  {
    uint16_t* dst = t < 128 ? sm.u.kq.Kr : sm.u.kq.Qr;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      *reinterpret_cast<u32x4_t*>(dst + sw128(8 * tb + j, 8 * gr)) = kv[j];
  }
  __syncthreads();

  // Gram tiles into registers.  Wave 0: the diagonal tiles of K K^T (so it
  // can invert T's diagonal blocks without waiting for others); wave 1: the
  // other tiles of K K^T; waves 2, 3: Q K^T.
  const uint16_t* Kr = sm.u.kq.Kr;
  const uint16_t* Qr = sm.u.kq.Qr;
  // The first value head of each key head also writes the chunk's K as the
  // scan's fragments, the second (or again the first, if it is alone) the
  // chunk's Q.  Wave w writes the four fragments of token tile w, read back
  // from the LDS tile in fragment order, so that every store of a wave
  // writes 1 KiB of whole lines.
  {
    const int sel = h % p.group;
    auto put = [&](const uint16_t* X, int mat) {
      uint4* dst = m.kqf + ((int64_t)q * p.h_k + hk) * kKqU4 + (mat * 16 + w * 4) * 64 + lane;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[j * 64] = *reinterpret_cast<const uint4*>(X + sw128(16 * w + c, 32 * j + 8 * g));
    };
    if (sel == 0) put(Kr, 0);
    if (sel == (p.group == 1 ? 0 : 1)) put(Qr, 1);
  }
  // Gates of the chunk (wave 0, whose Gram tiles are few), needed from the
  // epilogue on: log a and b in fp32, their chunk-local prefix sum in fp64
  // so that G_i - G_j keeps the small difference of two large sums.
  if (w == 0) {
    double ell = 0.0;
    float bb = 0.f;
    if (lane < L) {
      ell = (double)log_decay_f32(graw, direct ? 0.f : p.A_log[h],
                                  direct ? 0.f : p.dt_bias[h], direct);
      bb = write_strength_f32(braw, direct);
    }
    double G = ell;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    const double GL = __shfl(G, 63, 64);
    sm.G[lane] = G;
    sm.b[lane] = bb;
    float* gout = m.gate + ((int64_t)q * p.h_v + h) * 3 * kC;
    gout[lane] = expf((float)G);
    gout[kC + lane] = expf((float)(GL - G));
    gout[2 * kC + lane] = bb;
  }
  f32x4_t r0, r1, r2, r3, r4, r5;
  switch (w) {
    case 0:
      r0 = gram_t(Kr, Kr, 0, 0, g, c); r1 = gram_t(Kr, Kr, 1, 1, g, c);
      r2 = gram_t(Kr, Kr, 2, 2, g, c); r3 = gram_t(Kr, Kr, 3, 3, g, c);
      break;
    case 1:
      r0 = gram_t(Kr, Kr, 2, 0, g, c); r1 = gram_t(Kr, Kr, 2, 1, g, c);
      r2 = gram_t(Kr, Kr, 3, 0, g, c); r3 = gram_t(Kr, Kr, 3, 1, g, c);
      r4 = gram_t(Kr, Kr, 3, 2, g, c); r5 = gram_t(Kr, Kr, 1, 0, g, c); break;
    case 2:
      r0 = gram_t(Qr, Kr, 0, 0, g, c); r1 = gram_t(Qr, Kr, 1, 0, g, c);
      r2 = gram_t(Qr, Kr, 1, 1, g, c); r3 = gram_t(Qr, Kr, 3, 2, g, c);
      r4 = gram_t(Qr, Kr, 3, 3, g, c); break;
    default:
      r0 = gram_t(Qr, Kr, 2, 0, g, c); r1 = gram_t(Qr, Kr, 2, 1, g, c);
      r2 = gram_t(Qr, Kr, 2, 2, g, c); r3 = gram_t(Qr, Kr, 3, 0, g, c);
      r4 = gram_t(Qr, Kr, 3, 1, g, c); break;
  }
  __syncthreads();   // K and Q are dead: their LDS now holds A and T

  switch (w) {
    case 0:
      a_tile(sm, r0, 0, 0, g, c); a_tile(sm, r1, 1, 1, g, c);
      a_tile(sm, r2, 2, 2, g, c); a_tile(sm, r3, 3, 3, g, c);
      t_diag(sm, g, c);
      break;
    case 1:
      a_tile(sm, r0, 2, 0, g, c); a_tile(sm, r1, 2, 1, g, c);
      a_tile(sm, r2, 3, 0, g, c); a_tile(sm, r3, 3, 1, g, c);
      a_tile(sm, r4, 3, 2, g, c); a_tile(sm, r5, 1, 0, g, c); break;
    // P's tiles (0,1) and (2,3), right of the diagonal inside 32-wide
    // k-steps of P U, are zero.
    case 2: {
      const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
      p_frag(rec, p_vals(sm, r0, 0, 0, g, c), zero, 0, 0, lane);
      p_frag(rec, p_vals(sm, r1, 1, 0, g, c), p_vals(sm, r2, 1, 1, g, c), 1, 0, lane);
      p_frag(rec, p_vals(sm, r3, 3, 2, g, c), p_vals(sm, r4, 3, 3, g, c), 3, 1, lane);
      break;
    }
    default: {
      const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
      p_frag(rec, p_vals(sm, r0, 2, 0, g, c), p_vals(sm, r1, 2, 1, g, c), 2, 0, lane);
      p_frag(rec, p_vals(sm, r2, 2, 2, g, c), zero, 2, 1, lane);
      p_frag(rec, p_vals(sm, r3, 3, 0, g, c), p_vals(sm, r4, 3, 1, g, c), 3, 0, lane);
      break;
    }
  }
  __syncthreads();
  // T below the diagonal, one column block per wave.
  if (w == 1) t_column<0>(sm, g, c);
  else if (w == 2) t_column<1>(sm, g, c);
  else if (w == 3) t_column<2>(sm, g, c);
  __syncthreads();
  // T fragments of token tile w (blocks right of the diagonal are zero).
  const int nks = w < 2 ? 1 : 2;
  for (int ks = 0; ks < nks; ++ks) {
    const int f = frag_index(w, ks);
    const int col0 = 32 * ks + 8 * g;
    bf16x8_t hi8, lo8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float x = (col0 + j) < 16 * (w + 1) ? sm.u.at.T32[16 * w + c][col0 + j] : 0.f;
      const __bf16 hb = (__bf16)x;
      hi8[j] = hb;
      lo8[j] = (__bf16)(x - (float)hb);
    }
    rec[(f * 2 + 0) * 64 + lane] = __builtin_bit_cast(uint4, hi8);
    rec[(f * 2 + 1) * 64 + lane] = __builtin_bit_cast(uint4, lo8);
  }
}

// ----------------------------------------------------------------- scan --

// Per-lane addressing of one work item, fixed for its whole sequence.
struct ScanCtx {
  const uint4* rec0;        // first chunk record of this head
  int64_t rec_stride;       // uint4 between consecutive chunk records
  const float* gate0;       // first gate record of this head
  int64_t gate_stride;      // floats between consecutive gate records
  int rowo;                 // first of the lane's 4 output token rows
  int vr;                   // the lane's state row within the slice
};

// Output of the recurrent read-out: fp32 staging for the tail pass, or the
// final o in fp32 / bf16.
enum { kOutStage = 0, kOutF32 = 1, kOutBf16 = 2 };

// Stores the read-out of chunk ci (its first L tokens).  The staging form
// stores the lane's four values whole (one contiguous 1 KiB write per wave;
// rows past L are never read), at out_col + ci * out_stride in 16-byte
// units.
template <int OUT>
__device__ __forceinline__ void store_out(void* out_col, int64_t out_stride,
                                          f32x4_t o, int ci, int L, int rowo) {
  if constexpr (OUT == kOutStage) {
    static_cast<uint4*>(out_col)[ci * out_stride] = __builtin_bit_cast(uint4, o);
    return;
  }
  const int64_t ob = ((int64_t)ci * kC + rowo) * out_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rowo + i < L) {
      const int64_t oi = ob + i * out_stride;
      if constexpr (OUT == kOutBf16)
        static_cast<uint16_t*>(out_col)[oi] = (uint16_t)f32_to_bf16_bits(o[i]);
      else
        static_cast<float*>(out_col)[oi] = o[i];
    }
  }
}

// ----------------------------------------------------------------- scan --
// The state chain.  Each compute wave loads the K and Q fragments of its
// token tile straight from memory into registers, two chunks ahead (issued
// right after a chunk's first barrier, when its fragments are no longer
// needed, for the chunk after next: an L2 round trip under this load takes
// longer than one chunk).  A fifth wave stages the rest of every chunk's
// operands into LDS, also two chunks ahead: the T/P record as stored, the
// slice's V columns and the gate record, with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave-uniform LDS
// base + 16 l; counted by vmcnt).  Three chunk buffers: the loader fills
// buffer (ci+2) % 3 during chunk ci and waits for chunk ci+1's loads before
// the chunk's last barrier.  K and Q do not pass through LDS: staged
// there they would double the LDS traffic of the chunk (the copy in, then
// the fragment reads) and slow the LDS reads of the chain.
constexpr int kLwThreads = 320;

struct LwBuf {
  uint4 rec[kRecU4];                    // T and P fragments, lane-major
  uint16_t V[kC * kSliceRows];          // V slice [token][row]
  float gate[3 * kC];                   // e^G, e^{G_L-G}, b
};

struct LwLds {
  uint16_t Sh[kSliceRows * kD], Sl[kSliceRows * kD];
  uint16_t Kt[kD * kC];
  uint16_t Rh[kSliceRows * kC], Rl[kSliceRows * kC];
  uint16_t Uh[kSliceRows * kC], Ul[kSliceRows * kC];
  uint16_t Wh[kSliceRows * kC], Wl[kSliceRows * kC];
  LwBuf buf[3];
};
static_assert(sizeof(LwLds) <= 160 * 1024, "loader-wave scan LDS");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS address of a pointer into the workgroup's shared arrays: its low 32
// bits, taken without the null test of a generic-to-LDS conversion.
__device__ __forceinline__ lds_ptr_t lds_addr(const void* p) {
  return (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)p;
}
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_addr(lds_base), 16, 0, 0);
}
// Same, from a wave-uniform base plus a 32-bit per-lane byte offset, so the
// address is formed by the load itself (scalar base + vector offset) rather
// than by 64-bit vector arithmetic.
__device__ __forceinline__ void dma16_at(const char* base, uint32_t off,
                                         void* lds_base) {
  __builtin_amdgcn_global_load_lds(base + off, lds_addr(lds_base), 16, 0, 0);
}

// s_waitcnt immediate: at most n vector memory operations outstanding
// (vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt not waited for).
constexpr int wait_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

// Barrier for the loader wave: it writes LDS only through direct-to-LDS
// loads, whose completion it waits for explicitly; a fence here would make
// it wait for every load in flight.
__device__ __forceinline__ void raw_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Byte offsets of the loader lane's V loads within a full chunk (token
// 32 i + lane / 2, 8 of the slice's 16 columns), the same for every chunk.
struct LwOffs {
  uint32_t v[2];
};

__device__ __forceinline__ LwOffs lw_offsets(const PrefillParams& p, int lane) {
  LwOffs o;
  const uint32_t vrow = (uint32_t)p.h_v * kD * 2;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    o.v[i] = (uint32_t)(32 * i + (lane >> 1)) * vrow + 16u * (uint32_t)(lane & 1);
  return o;
}

// Direct-to-LDS loads one lw_stage issues (T/P record, V, gates), whatever
// the chunk length: the loader waits for an older chunk's loads with
// vmcnt(kStageLoads) while the newest chunk's are still in flight.
constexpr int kStageLoads = kRecU4 / 64 + 2 + 1;

// One chunk's LDS operands into a buffer (loader wave).  V rows past the end
// of a short chunk repeat its last token (finite values that meet b = 0 and
// are never stored).
__device__ __forceinline__ void lw_stage(LwBuf& B, const PrefillParams& p,
                                         const ScanCtx& x, const LwOffs& o,
                                         int64_t t_beg, int h, int v0, int ci,
                                         int L, int lane) {
  const int64_t t0 = t_beg + (int64_t)ci * kC;
  const char* rec = reinterpret_cast<const char*>(x.rec0 + ci * x.rec_stride);
#pragma unroll
  for (int f = 0; f < kRecU4 / 64; ++f) {
    // each 1 KiB step stays on the scalar base (the empty asm keeps the
    // compiler from folding it into a 64-bit per-lane address)
    const char* rb = rec + 1024 * f;
    asm volatile("" : "+s"(rb));
    dma16_at(rb, 16u * lane, B.rec + 64 * f);
  }
  if (L == kC) {
    const char* vb = static_cast<const char*>(p.v) + ((t0 * p.h_v + h) * kD + v0) * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16_at(vb, o.v[i], B.V + 32 * i * kSliceRows);
  } else {
    const uint16_t* vg = static_cast<const uint16_t*>(p.v);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = min(32 * i + (lane >> 1), L - 1);
      dma16(vg + ((t0 + tok) * p.h_v + h) * kD + v0 + 8 * (lane & 1),
            B.V + 32 * i * kSliceRows);
    }
  }
  if (lane < 48)
    dma16_at(reinterpret_cast<const char*>(x.gate0 + ci * x.gate_stride),
             16u * lane, B.gate);
}

// K and Q fragments of token tile w from a chunk's fragment record (rows
// past the end of a short chunk repeat its last token) into registers: lane
// (g, c) holds token 16 w + c, dims 32 ks + 8 g .. +8.  Each load is one
// contiguous 1 KiB read per wave: loading the same fragments straight from
// the [token][head][dim] rows touches 16 half lines per load, and those
// requests, not the bytes, are what the scan's memory path spends its time
// on.
__device__ __forceinline__ void load_kq(bf16x8_t (&kf)[4], bf16x8_t (&qf)[4],
                                        const uint4* kq, int w, int lane) {
  const uint4* kp = kq + (w * 4) * 64 + lane;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = __builtin_bit_cast(bf16x8_t, kp[ks * 64]);
    qf[ks] = __builtin_bit_cast(bf16x8_t, kp[16 * 64 + ks * 64]);
  }
}

// One chunk for token tile w: K and Q fragments in kf / qf, the other
// operands in LDS buffer B.  Once the fragments are used, loads those of
// fragment record kq_next into kf / qf.  Returns the lane's four outputs.
template <int W>
__device__ __forceinline__ f32x4_t lw_chunk(LwLds& sm, const LwBuf& B,
                                            f32x4_t (&acc)[2], const ScanCtx& x,
                                            int lane, bf16x8_t (&kf)[4],
                                            bf16x8_t (&qf)[4],
                                            const uint4* kq_next) {
  constexpr int w = W;
  const int g = lane >> 4, c = lane & 15;
  const int r = x.vr;
  constexpr int nks = w < 2 ? 1 : 2;
  bf16x8_t sh[4], slo[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    sh[ks] = ld8(sm.Sh, sw128(r, 32 * ks + 8 * g));
    slo[ks] = ld8(sm.Sl, sw128(r, 32 * ks + 8 * g));
  }
  const float4 eg4 = *reinterpret_cast<const float4*>(&B.gate[x.rowo]);
  const float4 bb4 = *reinterpret_cast<const float4*>(&B.gate[2 * kC + x.rowo]);
  const f32x4_t eg = {eg4.x, eg4.y, eg4.z, eg4.w};
  const f32x4_t bb = {bb4.x, bb4.y, bb4.z, bb4.w};
  __builtin_amdgcn_sched_barrier(0);
  f32x4_t X = {0.f, 0.f, 0.f, 0.f}, Y = {0.f, 0.f, 0.f, 0.f};
  f32x4_t X2 = {0.f, 0.f, 0.f, 0.f}, Y2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    X = mfma32(kf[ks], sh[ks], X);
    Y = mfma32(qf[ks], sh[ks], Y);
    X2 = mfma32(kf[ks], slo[ks], X2);
    Y2 = mfma32(qf[ks], slo[ks], Y2);
  }
  X += X2;
  Y += Y2;
  // K^T of the chunk into LDS, two tokens per 32-bit store: lanes c and
  // c ^ 1 hold tokens 2m and 2m+1 of the same 8 dims; a quad-perm swap gives
  // each the other's values, and one byte permute with a per-lane selector
  // builds (even dim: tokens 2m, 2m+1) on the even lane and (odd dim) on
  // the odd one.
  {
    const int odd = c & 1;
    const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 kw = __builtin_bit_cast(uint4, kf[ks]);
      const uint32_t mine[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(
            0, (int)mine[pi], kDppQuadXor1, 0xF, 0xF, true);
        const uint32_t pair = __builtin_amdgcn_perm(other, mine[pi], sel);
        const int dim = 32 * ks + 8 * g + 2 * pi + odd;
        *reinterpret_cast<uint32_t*>(&sm.Kt[sw64(dim, 16 * w + (c & ~1))]) = pair;
      }
    }
  }
  f32x4_t R, Oacc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float vv = bf16_bits_to_f32(B.V[(x.rowo + i) * kSliceRows + r]);
    R[i] = bb[i] * (vv - eg[i] * X[i]);
    Oacc[i] = eg[i] * Y[i];
  }
  store_split4(sm.Rh, sm.Rl, sw64(r, 16 * w + 4 * g), R);
  lds_barrier();
  load_kq(kf, qf, kq_next, w, lane);

  // U = T R; W = diag(e^{G_L - G}) U.
  f32x4_t U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks < nks) {
      const int f = frag_index(w, ks);
      const bf16x8_t th = __builtin_bit_cast(bf16x8_t, B.rec[(f * 2 + 0) * 64 + lane]);
      const bf16x8_t tl = __builtin_bit_cast(bf16x8_t, B.rec[(f * 2 + 1) * 64 + lane]);
      const bf16x8_t rh = ld8(sm.Rh, sw64(r, 32 * ks + 8 * g));
      const bf16x8_t rl = ld8(sm.Rl, sw64(r, 32 * ks + 8 * g));
      U = mfma32(th, rh, U);
      U = mfma32(th, rl, U);
      U = mfma32(tl, rh, U);
    }
  }
  const float4 egl4 = *reinterpret_cast<const float4*>(&B.gate[kC + x.rowo]);
  const float eL = B.gate[kC - 1];
  store_split4(sm.Uh, sm.Ul, sw64(r, 16 * w + 4 * g), U);
  store_split4(sm.Wh, sm.Wl, sw64(r, 16 * w + 4 * g),
               f32x4_t{egl4.x, egl4.y, egl4.z, egl4.w} * U);
  lds_barrier();

  // O = diag(e^G) Q S0^T + P U.
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    if (ks < nks) {
      const int f = frag_index(w, ks);
      const bf16x8_t ph = __builtin_bit_cast(bf16x8_t, B.rec[((kFrags + f) * 2 + 0) * 64 + lane]);
      const bf16x8_t pl = __builtin_bit_cast(bf16x8_t, B.rec[((kFrags + f) * 2 + 1) * 64 + lane]);
      const bf16x8_t uh = ld8(sm.Uh, sw64(r, 32 * ks + 8 * g));
      const bf16x8_t ul = ld8(sm.Ul, sw64(r, 32 * ks + 8 * g));
      Oacc = mfma32(ph, uh, Oacc);
      Oacc = mfma32(ph, ul, Oacc);
      Oacc = mfma32(pl, uh, Oacc);
    }
  }
  // S^T <- e^{G_L} S^T + K^T W on dim tiles 2w, 2w+1.
#pragma unroll
  for (int dl = 0; dl < 2; ++dl) {
    acc[dl] *= eL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t a = ld8(sm.Kt, sw64(16 * (2 * w + dl) + c, 32 * ks + 8 * g));
      const bf16x8_t bh = ld8(sm.Wh, sw64(r, 32 * ks + 8 * g));
      const bf16x8_t bl = ld8(sm.Wl, sw64(r, 32 * ks + 8 * g));
      acc[dl] = mfma32(a, bh, acc[dl]);
      acc[dl] = mfma32(a, bl, acc[dl]);
    }
    store_split4(sm.Sh, sm.Sl, sw128(r, 16 * (2 * w + dl) + 4 * g), acc[dl]);
  }
  lds_barrier();
  return Oacc;
}

// The compute waves' part of the scan; the wave index is a template
// parameter, so each wave's chain is straight-line code (its k-step counts
// and fragment choices resolved at compile time).
template <int OUT, int W>
__device__ __forceinline__ void scan_compute(LwLds& sm, const PrefillParams& p,
                                             const Maps& m, const ScanCtx& x, int lane,
                                             int q0, int h, int hk, int sl, int v0,
                                             int64_t t_beg, int64_t len, int nch,
                                             int64_t srow) {
  constexpr int w = W;
  const int g = lane >> 4;
  auto chunk_len = [&](int ci) -> int {
    const int64_t r = len - (int64_t)ci * kC;
    return (int)(r < kC ? r : kC);
  };
  void* out_col;
  int64_t out_stride = (int64_t)p.h_v * kD;
  const int64_t ocol = (t_beg * p.h_v + h) * kD + v0 + x.vr;
  if constexpr (OUT == kOutStage) {
    out_col = m.stage + (((int64_t)q0 * p.h_v + h) * kSlices + sl) * 256 + w * 64 + lane;
    out_stride = (int64_t)p.h_v * kSlices * 256;
  } else if constexpr (OUT == kOutF32) {
    out_col = static_cast<float*>(p.out) + ocol;
  } else {
    out_col = static_cast<uint16_t*>(p.out) + ocol;
  }

  f32x4_t acc[2];
#pragma unroll
  for (int dl = 0; dl < 2; ++dl) {
    const int col = 16 * (2 * w + dl) + 4 * g;
    if (p.s0) {
      const float4 v = *reinterpret_cast<const float4*>(p.s0 + srow + col);
      acc[dl] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      acc[dl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    store_split4(sm.Sh, sm.Sl, sw128(x.vr, col), acc[dl]);
  }
  lds_barrier();

  // K / Q fragments two chunks ahead in two register sets, used by
  // alternate chunks (the loop runs chunk 0, then pairs).  Every load and
  // store of the loop is unconditional, so the compiler's count of memory
  // operations in flight is exact and the wait before a chunk's first
  // product covers only that chunk's fragments.  Past the last chunk the
  // loads read the last chunk again (a valid address; never used).
  const uint4* kq0 = m.kqf + ((int64_t)q0 * p.h_k + hk) * kKqU4;
  const int64_t kq_stride = (int64_t)p.h_k * kKqU4;
  auto ahead = [&](int ci) { return kq0 + (ci < nch ? ci : nch - 1) * kq_stride; };
  bf16x8_t kf[4], qf[4], kf2[4], qf2[4];
  load_kq(kf, qf, kq0, w, lane);
  load_kq(kf2, qf2, ahead(1), w, lane);
  f32x4_t o_prev = lw_chunk<W>(sm, sm.buf[0], acc, x, lane, kf, qf, ahead(2));
  // (The loop has no early exit: a path from the middle of the body to its
  // head would make the compiler assume the second half's loads may be
  // missing and wait for the newest fragments too.)
  int bi = 1, ci = 1;
  for (; ci + 1 < nch; ci += 2) {
    store_out<OUT>(out_col, out_stride, o_prev, ci - 1, kC, x.rowo);
    o_prev = lw_chunk<W>(sm, sm.buf[bi], acc, x, lane, kf2, qf2, ahead(ci + 2));
    bi = bi == 2 ? 0 : bi + 1;
    store_out<OUT>(out_col, out_stride, o_prev, ci, kC, x.rowo);
    o_prev = lw_chunk<W>(sm, sm.buf[bi], acc, x, lane, kf, qf, ahead(ci + 3));
    bi = bi == 2 ? 0 : bi + 1;
  }
  if (ci < nch) {
    store_out<OUT>(out_col, out_stride, o_prev, ci - 1, kC, x.rowo);
    o_prev = lw_chunk<W>(sm, sm.buf[bi], acc, x, lane, kf2, qf2, ahead(ci + 2));
  }
  store_out<OUT>(out_col, out_stride, o_prev, nch - 1, chunk_len(nch - 1), x.rowo);

  if (p.sF) {
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
      const int col = 16 * (2 * w + dl) + 4 * g;
      *reinterpret_cast<float4*>(p.sF + srow + col) =
          make_float4(acc[dl][0], acc[dl][1], acc[dl][2], acc[dl][3]);
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(kLwThreads) void scan_lw_kernel(PrefillParams p,
                                                             Maps m) {
  __shared__ LwLds sm;
  const int t = threadIdx.x;
  // The wave index as a scalar: branches on it (loader wave, per-wave code)
  // are uniform, and each wave runs only its own barriers.
  const int lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;

  const int nb = gridDim.x;
  const int lid = (nb & 7) == 0 ? (blockIdx.x & 7) * (nb >> 3) + (blockIdx.x >> 3)
                                : blockIdx.x;
  const int sl = lid % kSlices;
  const int nh = lid / kSlices;
  const int n = nh / p.h_v;
  const int h = nh - n * p.h_v;
  const int hk = h / p.group;
  const int v0 = sl * kSliceRows;
  int64_t t_beg, t_end;
  seq_range(p, n, t_beg, t_end);
  const int q0 = m.prefix[n];
  const int nch = m.prefix[n + 1] - q0;
  const int64_t len = t_end - t_beg;
  auto chunk_len = [&](int ci) -> int {
    const int64_t r = len - (int64_t)ci * kC;
    return (int)(r < kC ? r : kC);
  };

  ScanCtx x;
  x.vr = c;
  x.rowo = 16 * (w & 3) + 4 * g;
  x.rec_stride = (int64_t)p.h_v * kRecU4;
  x.rec0 = m.rec + ((int64_t)q0 * p.h_v + h) * kRecU4;
  x.gate_stride = (int64_t)p.h_v * 3 * kC;
  x.gate0 = m.gate + ((int64_t)q0 * p.h_v + h) * 3 * kC;

  const int64_t srow = ((int64_t)nh * kD + v0 + x.vr) * kD;
  if (nch == 0) {
    // Empty sequence: the final state is the initial one.
    if (w < 4 && p.sF) {
#pragma unroll
      for (int dl = 0; dl < 2; ++dl) {
        const int col = 16 * (2 * w + dl) + 4 * g;
        const float4 v = p.s0 ? *reinterpret_cast<const float4*>(p.s0 + srow + col)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(p.sF + srow + col) = v;
      }
    }
    return;
  }

  if (w == 4) {
    // Loader wave, two chunks ahead over three buffers: chunks 0 and 1
    // before the first barrier, then chunk ci+2 during chunk ci; one barrier
    // for each of the compute waves'.  Before the barrier that ends chunk ci
    // it waits for chunk ci+1's loads, leaving chunk ci+2's in flight.
    const LwOffs o = lw_offsets(p, lane);
    lw_stage(sm.buf[0], p, x, o, t_beg, h, v0, 0, chunk_len(0), lane);
    if (nch > 1) lw_stage(sm.buf[1], p, x, o, t_beg, h, v0, 1, chunk_len(1), lane);
    __builtin_amdgcn_sched_barrier(0);
    if (nch > 1) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kStageLoads));
    else __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
    raw_barrier();
    int bs = 2;
    for (int ci = 0; ci < nch; ++ci) {
      if (ci + 2 < nch)
        lw_stage(sm.buf[bs], p, x, o, t_beg, h, v0, ci + 2, chunk_len(ci + 2), lane);
      raw_barrier();
      raw_barrier();
      __builtin_amdgcn_sched_barrier(0);
      if (ci + 2 < nch) __builtin_amdgcn_s_waitcnt(wait_vmcnt(kStageLoads));
      else __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
      raw_barrier();
      bs = bs == 2 ? 0 : bs + 1;
    }
    return;
  }

  switch (w) {
    case 0: scan_compute<OUT, 0>(sm, p, m, x, lane, q0, h, hk, sl, v0, t_beg, len, nch, srow); break;
    case 1: scan_compute<OUT, 1>(sm, p, m, x, lane, q0, h, hk, sl, v0, t_beg, len, nch, srow); break;
    case 2: scan_compute<OUT, 2>(sm, p, m, x, lane, q0, h, hk, sl, v0, t_beg, len, nch, srow); break;
    default: scan_compute<OUT, 3>(sm, p, m, x, lane, q0, h, hk, sl, v0, t_beg, len, nch, srow); break;
  }
}

// ----------------------------------------------------------------- tail --
// Gated RMSNorm ("Red Lite dev15d -- DeltaNet gated tail + Q4_K output
// projection", Pinned graph semantics steps 2-5) over the scan's blocked
// read-out: one workgroup per (chunk slot, value head).  Wave w takes token
// tile w.  Lane (g, c) reads, for each slice s, the four tokens 16 w + 4 g ..
// +3 of column 16 s + c exactly as the scan's lane stored them (contiguous
// 1 KiB reads), sums their squares over its 8 columns and then over the 16
// lanes of its row group, and writes x * rsqrt(mean x^2 + eps) * w to LDS;
// it then reads the tile back by token rows (columns 4 c .. +3 and 64 + 4 c
// .. +3 of token 16 w + g + 4 j) to multiply by SiLU(z) and store the
// head-major output row with coalesced accesses.
constexpr int kTailLd = 132;

template <bool BF16>
__device__ __forceinline__ f32x4_t load4(const void* base, int64_t idx) {
  if constexpr (BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return f32x4_t{bf16_bits_to_f32(u.x & 0xffffu), bf16_bits_to_f32(u.x >> 16),
                   bf16_bits_to_f32(u.y & 0xffffu), bf16_bits_to_f32(u.y >> 16)};
  } else {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    return f32x4_t{v.x, v.y, v.z, v.w};
  }
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t idx, f32x4_t v) {
  if constexpr (BF16) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) =
        make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <bool ZB, bool OB>
__global__ __launch_bounds__(256) void tail_kernel(PrefillParams p, Maps m) {
  __shared__ float ys[4][16][kTailLd];
  const int q = blockIdx.x / p.h_v, h = blockIdx.x - q * p.h_v;
  const int n = m.chunk_seq[q];
  if (n < 0) return;
  int64_t s_beg, s_end;
  seq_range(p, n, s_beg, s_end);
  const int64_t t0 = s_beg + (int64_t)(q - m.prefix[n]) * kC;
  const int L = (int)((s_end - t0) < kC ? (s_end - t0) : kC);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;

  // z of the lane's output rows (rows past the end of a short chunk read
  // its last token; they are not stored).
  f32x4_t za[4], zb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = min(16 * w + g + 4 * j, L - 1);
    const int64_t zr = ((t0 + tok) * p.h_v + h) * kD;
    za[j] = load4<ZB>(p.z, zr + 4 * c);
    zb[j] = load4<ZB>(p.z, zr + 64 + 4 * c);
  }
  const uint4* blk = m.stage + (int64_t)blockIdx.x * kSlices * 256 + w * 64 + lane;
  f32x4_t v[kSlices];
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl)
    v[sl] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(blk + sl * 256));
  float wt[kSlices];
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl) wt[sl] = p.w[16 * sl + c];
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int sl = 0; sl < kSlices; ++sl) ss += v[sl][i] * v[sl][i];
    ss = group_sum<16>(ss);
    inv[i] = rsqrtf(ss / (float)kD + p.eps);
  }
#pragma unroll
  for (int sl = 0; sl < kSlices; ++sl)
#pragma unroll
    for (int i = 0; i < 4; ++i) ys[w][4 * g + i][16 * sl + c] = v[sl][i] * inv[i] * wt[sl];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = g + 4 * j, tok = 16 * w + row;
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(&ys[w][row][4 * c]);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&ys[w][row][64 + 4 * c]);
    f32x4_t ya, yb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ya[i] = a[i] * silu_f32(za[j][i]);
      yb[i] = b[i] * silu_f32(zb[j][i]);
    }
    if (tok < L) {
      const int64_t orow = ((t0 + tok) * p.h_v + h) * kD;
      store4<OB>(p.out, orow + 4 * c, ya);
      store4<OB>(p.out, orow + 64 + 4 * c, yb);
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t prefix, chunk_seq, rec, kqf, gate, stage, total;
  int32_t QB;
};

WsLayout ws_layout(int64_t T, int32_t N, int32_t h_k, int32_t h_v,
                   int32_t d_v, bool tail) {
  WsLayout l;
  l.QB = (int32_t)(T / kC + N);
  size_t off = 0;
  l.prefix = off;    off += align256(sizeof(int32_t) * (N + 1));
  l.chunk_seq = off; off += align256(sizeof(int32_t) * (size_t)l.QB);
  l.rec = off;       off += align256(sizeof(uint4) * (size_t)l.QB * h_v * kRecU4);
  l.kqf = off;       off += align256(sizeof(uint4) * (size_t)l.QB * h_k * kKqU4);
  l.gate = off;      off += align256(sizeof(float) * (size_t)l.QB * h_v * 3 * kC);
  l.stage = off;     off += tail ? align256(sizeof(float) * (size_t)l.QB * kC * h_v * d_v) : 0;
  l.total = off;
  return l;
}

}  // namespace

Bf16Plan plan_prefill_bf16(int64_t T, int32_t N, int32_t h_k, int32_t h_v,
                           int32_t d_v, bool tail) {
  Bf16Plan plan;
  plan.slices = kSlices;
  plan.ws_bytes = ws_layout(T, N, h_k, h_v, d_v, tail).total;
  return plan;
}

hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream) {
  const WsLayout l = ws_layout(p.T, p.N, p.h_k, p.h_v, p.d_v, p.tail != 0);
  char* base = reinterpret_cast<char*>(p.ws);
  Maps m;
  m.prefix = reinterpret_cast<int32_t*>(base + l.prefix);
  m.chunk_seq = reinterpret_cast<int32_t*>(base + l.chunk_seq);
  m.rec = reinterpret_cast<uint4*>(base + l.rec);
  m.kqf = reinterpret_cast<uint4*>(base + l.kqf);
  m.gate = reinterpret_cast<float*>(base + l.gate);
  m.stage = p.tail ? reinterpret_cast<uint4*>(base + l.stage) : nullptr;
  m.QB = l.QB;
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, stream, p, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (l.QB > 0) {
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)((int64_t)l.QB * p.h_v)),
                       dim3(kThreads), 0, stream, p, m);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t blocks = (int64_t)p.N * p.h_v * kSlices;
  if (blocks > 0) {
    const int mode = p.tail ? kOutStage : (p.out_bf16 ? kOutBf16 : kOutF32);
    if (mode == kOutStage)
      hipLaunchKernelGGL(scan_lw_kernel<kOutStage>, dim3((unsigned)blocks),
                         dim3(kLwThreads), 0, stream, p, m);
    else if (mode == kOutF32)
      hipLaunchKernelGGL(scan_lw_kernel<kOutF32>, dim3((unsigned)blocks),
                         dim3(kLwThreads), 0, stream, p, m);
    else
      hipLaunchKernelGGL(scan_lw_kernel<kOutBf16>, dim3((unsigned)blocks),
                         dim3(kLwThreads), 0, stream, p, m);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.tail && p.T > 0) {
    const dim3 grid((unsigned)((int64_t)l.QB * p.h_v));
    if (p.io_bf16 && p.out_bf16)
      hipLaunchKernelGGL((tail_kernel<true, true>), grid, dim3(256), 0, stream, p, m);
    else if (p.io_bf16)
      hipLaunchKernelGGL((tail_kernel<true, false>), grid, dim3(256), 0, stream, p, m);
    else if (p.out_bf16)
      hipLaunchKernelGGL((tail_kernel<false, true>), grid, dim3(256), 0, stream, p, m);
    else
      hipLaunchKernelGGL((tail_kernel<false, false>), grid, dim3(256), 0, stream, p, m);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdn
