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
// Three launches:
//  1. chunk_map: per-sequence chunk offsets (from cu_seqlens) and the
//     sequence of every chunk slot, longest sequences first.
//  2. prep (one workgroup per chunk and value head, fully parallel): the
//     gates, the Grams K K^T and Q K^T, P and T = (I + A)^{-1} -- everything
//     that does not depend on the state.  T and P are written as hi/lo bf16
//     matrix-core fragments, and the chunk's K and Q, once per key head, as
//     the fragments the scan loads (one contiguous 1 KiB read per load).
//  3. scan (one workgroup per sequence, value head and 16-row slice of the
//     state): the state-dependent chain only, chunk after chunk, with the
//     16 x 128 fp32 state slice resident in the matrix-core accumulators.
//     Per chunk: K S0^T, R; Q S0^T, T R; the state update -- three
//     barriers.  Chain waves load their K / Q fragments two chunks ahead; a
//     loader wave stages V, gates and z into LDS with direct-to-LDS loads.
//     With z, the scan also applies the gated RMSNorm: the 8 slices of a
//     head exchange per-token sums of squares a few chunks behind, and an
//     output wave writes the normalised, gated output head-major.
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
#include "gdn_seqmap.h"

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
// stored hi then lo.  A chunk record holds T's then P's.  (kMatU4 below.)
// Two of them lie partly right of the diagonal block -- f = 0 (token tile 0)
// and f = 3 (tile 2, second k-step): their lanes 32..63 (columns 16..31 of
// the k-step) are zero, so the record keeps lanes 0..31 only and the scan
// sets the others to zero.  Fragment f's hi part starts at
// frag_base(f) in its matrix, its lo part frag_lanes(f) later.
constexpr bool frag_half(int f) { return f == 0 || f == 3; }
constexpr int frag_lanes(int f) { return frag_half(f) ? 32 : 64; }
constexpr int frag_base(int f) {
  return f == 0 ? 0 : f == 1 ? 64 : f == 2 ? 192 : f == 3 ? 320 : f == 4 ? 384 : 512;
}
constexpr int kMatU4 = 640;                    // uint4 per matrix (T or P)
constexpr int kRecU4 = 2 * kMatU4;             // uint4 per chunk record
// K and Q of one chunk and key head as matrix-core fragments: fragment
// (token tile w, k-step ks) is 64 lanes x 16 bytes, lane (g, c) holding
// token 16 w + c, dims 32 ks + 8 g .. +7.  K's 16 fragments, then Q's.
constexpr int kKqU4 = 2 * 16 * 64;
// Exchange slots of the gated tail per chunk and value head: the 8 slices'
// sums of squares of each token, then their total.
constexpr int kSlots = 9;
__device__ __forceinline__ int frag_index(int w, int ks) {
  return w < 2 ? w : 2 * w - 2 + ks;
}

__device__ __forceinline__ int sw128(int r, int c) {
  return r * 128 + ((((c >> 3) ^ (r & 15)) << 3) | (c & 7));
}
// The scan's K tile: the same layout with the 16-byte pieces of row r
// permuted by f(r) = 2 (r % 4) + (r / 4) % 2 + 8 ((r / 8) % 2), so that both
// its writes (16 rows, one piece) and its transposing reads (4 rows, two
// adjacent pieces, in two row groups 8 apart) hit distinct banks.
__device__ __forceinline__ int sw128k(int r, int c) {
  const int f = ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);
  return r * 128 + ((((c >> 3) ^ f) << 3) | (c & 7));
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
  int32_t* seq_beg;    // [N] first token of each sequence (clamped)
  int32_t* seq_end;    // [N] one past its last token (clamped)
  int32_t* seq_order;  // [N] sequences by decreasing length (scan order)
  int32_t* chunk_seq;  // [QB] sequence of each chunk slot, -1 if unused
  uint4* rec;          // [QB][h_v][kRecU4] T and P fragments
  uint4* kqf;          // [QB][h_k][kKqU4] K and Q fragments
  float* gate;         // [QB][h_v][3][64]: e^G, e^{G_L - G}, b
  // Gated tail: each slice's sum of squares of the read-out over its 16
  // columns, then their total, [QB][h_v][9][64 tokens]; -1 until stored.
  float* part;
  int32_t QB;
};

// Token range of sequence n as laid out by the chunk map.
__device__ __forceinline__ void seq_range(const Maps& m, int n, int64_t& beg,
                                          int64_t& end) {
  beg = m.seq_beg[n];
  end = m.seq_end[n];
}

// ------------------------------------------------------------ chunk map --
// Sequence ranges from cu_seqlens, clamped into disjoint ranges inside
// [0, T] (so no later kernel can index past T or past the QB chunk slots,
// whatever the device offsets hold), the first chunk slot of each sequence,
// the sequence of every chunk slot, and the scan's order of sequences:
// longest first, so that the longest chains start first.
constexpr int kMaxOrdered = 4096;   // more sequences keep their own order

__global__ __launch_bounds__(256) void chunk_map_kernel(PrefillParams p,
                                                        Maps m) {
  if (threadIdx.x == 0)
    seq_layout(p.cu, p.N, p.seq_len, p.T, kC, m.seq_beg, m.seq_end, m.prefix);
  __syncthreads();
  for (int n = threadIdx.x; n < p.N; n += 256) {
    int rank = n;
    if (p.N <= kMaxOrdered) {
      const int32_t len = m.seq_end[n] - m.seq_beg[n];
      rank = 0;
      for (int j = 0; j < p.N; ++j) {
        const int32_t lj = m.seq_end[j] - m.seq_beg[j];
        rank += (lj > len) || (lj == len && j < n);
      }
    }
    m.seq_order[rank] = n;
  }
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
  const uint4 hi = tiles_to_frag(ah, bh), lo = tiles_to_frag(al, bl);
  if (lane < frag_lanes(f)) {
    uint4* at = rec + kMatU4 + frag_base(f) + lane;
    at[0] = hi;
    at[frag_lanes(f)] = lo;
  }
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
  seq_range(m, n, s_beg, s_end);
  const int64_t t0 = s_beg + (int64_t)(q - m.prefix[n]) * kC;
  const int L = (int)((s_end - t0) < kC ? (s_end - t0) : kC);
  const bool direct = p.direct != 0;
  uint4* rec = m.rec + ((int64_t)q * p.h_v + h) * kRecU4;
  // The gated tail's sum slots of this chunk and head start as -1 (absent).
  if (m.part) {
    float* pb = m.part + ((int64_t)q * p.h_v + h) * kSlots * kC;
    for (int i = threadIdx.x; i < kSlots * kC; i += kThreads) pb[i] = -1.f;
  }

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
    if (lane < frag_lanes(f)) {
      uint4* at = rec + frag_base(f) + lane;
      at[0] = __builtin_bit_cast(uint4, hi8);
      at[frag_lanes(f)] = __builtin_bit_cast(uint4, lo8);
    }
  }
}

// ----------------------------------------------------------------- scan --
// One workgroup per (sequence, value head, 16-row slice of the state) and
// eleven waves: four chain waves (0-3), four state waves (4-7), a loader
// (8), and an exchange (9) and an output wave (10) for the gated tail.
// Chain wave w and state wave 4 + w share a SIMD; chain wave w owns token
// tile w (tokens 16 w .. 16 w + 15) of every chunk, state wave 4 + j owns
// dimension tiles 2 j, 2 j + 1 of the slice's state S^T, held in
// matrix-core accumulators for the whole sequence.  Per chunk, with S0 the state entering it:
//   phase A  chain: X = K S0^T (S0 as hi / lo bf16 from LDS);
//                   R = diag(b) (V - diag(e^G) X) as hi / lo into LDS; K
//                   into LDS
//            state: O of the previous chunk = diag(e^G) Y + P U, stored
//                   (gated tail: kept in LDS); S^T *= e^{G_L}
//   -- barrier 1 --
//   phase B  chain: Y = Q S0^T (its products fill the matrix core while the
//                   R reads are in flight); U = T R; W = diag(e^{G_L - G}) U
//                   and U as hi / lo, and Y into LDS
//            loader: V and gates of the chunk after next into LDS
//   -- barrier 2 --
//   phase C  state: S^T += K^T W (K^T read from the K tile with the LDS
//                   transpose read); S as hi / lo into LDS (next S0)
//            exchange: (gated tail) sums of squares across the slices
//            chain: prefetch (the K fragments at the end of phase A); (gated
//                   tail) w * SiLU(z) of an earlier chunk
//   -- barrier 3 --
// The chain waves' phases A, B and the state waves' phase C are the serial
// chain; the read-out runs beside it on the other wave of each SIMD.
//
// Memory: every vector-memory instruction costs the compute unit's load
// path about the same whatever its width, so operands arrive as whole
// 1 KiB loads (16 bytes per lane): the chain waves load the K, Q and T
// fragments that prep wrote in lane order, the state waves the P
// fragments, each into registers, ahead of use; the loader wave stages each
// chunk's V slice and gate record into LDS rings with direct-to-LDS loads
// (three loads per chunk instead of gathers on every compute wave).  K^T
// is never loaded: the chain waves store their K fragments in an LDS tile
// and the state waves read them transposed.  Every load and store of the
// chunk loops is unconditional (past the last chunk they repeat it), so the
// compiler's count of memory operations in flight is exact.
constexpr int kScanThreads = 704;

// Output of the scan: o itself (fp32 / bf16), or the gated RMSNorm of o
// (fp32 / bf16), computed in the scan.
enum { kOutF32 = 0, kOutBf16 = 1, kOutGatedF32 = 2, kOutGatedBf16 = 3 };
constexpr bool is_gated(int out) { return out >= kOutGatedF32; }
constexpr bool out_is_bf16(int out) { return (out & 1) != 0; }

// Row stride (floats) of the gated tail's read-out ring: the state waves'
// column-wise writes (row 4 g + i, column c) and the loader's row reads (a
// 16-lane pass reading rows t .. t + 15) both hit distinct banks.
constexpr int kOtLd = 20;

struct ScanLds {
  uint16_t Sh[kSliceRows * kD], Sl[kSliceRows * kD];   // S0 hi / lo [row][dim]
  uint16_t Kb[kC * kD];                                // K [token][dim] (sw128k)
  uint16_t Rh[kSliceRows * kC], Rl[kSliceRows * kC];   // R^T [row][token]
  uint16_t Uh[kSliceRows * kC], Ul[kSliceRows * kC];   // U^T
  uint16_t Wh[kSliceRows * kC], Wl[kSliceRows * kC];   // W^T
  f32x4_t Y[4][64];                                    // Y, lane order
  uint16_t V[3][kC * kSliceRows];                      // V slice [token][row]
  float gate[3][3 * kC];                               // e^G, e^{G_L-G}, b
  // Gated tail (rings indexed by chunk % 8): read-outs awaiting their
  // normalisers, [token][column] with rows of kOtLd floats; z slices
  // (staged with V); 1 / RMS of each token.
  float Ot[8][kC * kOtLd];
  uint16_t Z[8][kC * kSliceRows];
  float rstd[8][kC];
  // w * SiLU(z) per token and column of the slice, and w itself.
  float Gz[8][kC * kSliceRows];
  float wn[kSliceRows];
};
static_assert(sizeof(ScanLds) <= 144 * 1024, "scan LDS");

// Addressing of one work item, fixed for its whole sequence.
struct ScanCtx {
  const uint4* kq0;         // K / Q record of the first chunk (key head)
  int64_t kq_stride;        // uint4 between consecutive chunks' records
  const uint4* rec0;        // T / P record of the first chunk (value head)
  int64_t rec_stride;
  const float* gate0;       // gate record of the first chunk
  int64_t gate_stride;
  int64_t len;              // tokens of the sequence
  int nch;                  // chunks of the sequence
};

__device__ __forceinline__ int clamp_chunk(const ScanCtx& x, int ci) {
  return ci < x.nch ? ci : x.nch - 1;
}

// Splits four fp32 values into hi = rne(x) and lo = rne(x - hi), packed as
// bf16 pairs (hi from one packed conversion per pair; its halves widened
// by shifts).
__device__ __forceinline__ void split4p(f32x4_t x, uint2& hi, uint2& lo) {
  const uint32_t h01 = pack_bf16x2(x[0], x[1]), h23 = pack_bf16x2(x[2], x[3]);
  const float f0 = __uint_as_float(h01 << 16), f1 = __uint_as_float(h01 & 0xffff0000u);
  const float f2 = __uint_as_float(h23 << 16), f3 = __uint_as_float(h23 & 0xffff0000u);
  hi = make_uint2(h01, h23);
  lo = make_uint2(pack_bf16x2(x[0] - f0, x[1] - f1), pack_bf16x2(x[2] - f2, x[3] - f3));
}
__device__ __forceinline__ void store_split4p(uint16_t* hi_arr, uint16_t* lo_arr,
                                              int off, f32x4_t x) {
  uint2 h, l;
  split4p(x, h, l);
  *reinterpret_cast<uint2*>(hi_arr + off) = h;
  *reinterpret_cast<uint2*>(lo_arr + off) = l;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// LDS address of a pointer into the workgroup's shared arrays: its low 32
// bits, taken without the null test of a generic-to-LDS conversion.
__device__ __forceinline__ lds_ptr_t lds_addr(const void* p) {
  return (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)p;
}
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_addr(lds_base), 16, 0, 0);
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

// K^T fragment (dimension tile d, token k-step ks) from the K tile: lane
// (g, c) receives K[32 ks + 8 g + i][16 d + c], i = 0..7.  The transpose
// read hands lane m of each 16-lane group element m % 4 of the 4-element
// pieces addressed by lanes m / 4 + 4 j (j = 0..3); so lane m addresses
// token t0 + m / 4 at dimensions 16 d + 4 (m % 4) .. +3, and two reads
// (t0 = 32 ks + 8 g and t0 + 4) give the eight values.
__device__ __forceinline__ bf16x8_t kt_frag(const uint16_t* Kb, int d, int ks,
                                            int lane) {
  const int g = lane >> 4, m = lane & 15;
  const int t0 = 32 * ks + 8 * g + (m >> 2);
  const int col = 16 * d + 4 * (m & 3);
  const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)lds_addr(Kb + sw128k(t0, col)));
  const bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4_t*)lds_addr(Kb + sw128k(t0 + 4, col)));
  return bf16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int W>
struct ChainOps {
  static constexpr int nks = W < 2 ? 1 : 2;   // k-steps of T R and P U
  bf16x8_t kf[4], qf[4];                      // K, Q fragments of tile W
};
template <int W>
struct TOps {
  bf16x8_t th[ChainOps<W>::nks], tl[ChainOps<W>::nks];
};

// K (Q) fragments of token tile W of chunk ci.
template <int W>
__device__ __forceinline__ void load_k(ChainOps<W>& o, const ScanCtx& x, int ci, int lane) {
  ci = clamp_chunk(x, ci);
  const uint4* kq = x.kq0 + ci * x.kq_stride + lane;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) o.kf[ks] = __builtin_bit_cast(bf16x8_t, kq[(W * 4 + ks) * 64]);
}
template <int W>
__device__ __forceinline__ void load_q(ChainOps<W>& o, const ScanCtx& x, int ci, int lane) {
  ci = clamp_chunk(x, ci);
  const uint4* kq = x.kq0 + ci * x.kq_stride + lane;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    o.qf[ks] = __builtin_bit_cast(bf16x8_t, kq[(16 + W * 4 + ks) * 64]);
}
template <int W>
__device__ __forceinline__ void load_kq(ChainOps<W>& o, const ScanCtx& x, int ci,
                                        int lane) {
  load_k<W>(o, x, ci, lane);
  load_q<W>(o, x, ci, lane);
}

// T (sel 0) or P (sel 1) fragments of token tile W, hi and lo.
template <int W>
__device__ __forceinline__ void load_tp(TOps<W>& o, const ScanCtx& x, int ci,
                                        int sel, int lane) {
  ci = clamp_chunk(x, ci);
  const uint4* mat = x.rec0 + ci * x.rec_stride + sel * kMatU4;
#pragma unroll
  for (int ks = 0; ks < ChainOps<W>::nks; ++ks) {
    const int f = frag_index(W, ks);
    // A stored half is read by all 64 lanes (lanes 32..63 repeat lanes
    // 0..31's lines) and the upper lanes then take zero.
    const int l = frag_half(f) ? (lane & 31) : lane;
    uint4 hi = mat[frag_base(f) + l], lo = mat[frag_base(f) + frag_lanes(f) + l];
    if (frag_half(f) && lane >= 32) hi = lo = make_uint4(0u, 0u, 0u, 0u);
    o.th[ks] = __builtin_bit_cast(bf16x8_t, hi);
    o.tl[ks] = __builtin_bit_cast(bf16x8_t, lo);
  }
}

// Stores the lane's four values of chunk ci (rows rowo .. +3 of the chunk,
// those below L) at out_col + (ci * 64 + row) * out_stride.
template <int OUT>
__device__ __forceinline__ void store_out(void* out_col, int64_t out_stride,
                                          f32x4_t o, int ci, int L, int rowo) {
  const int64_t ob = ((int64_t)ci * kC + rowo) * out_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (rowo + i < L) {
      const int64_t oi = ob + i * out_stride;
      if constexpr (out_is_bf16(OUT))
        static_cast<uint16_t*>(out_col)[oi] = (uint16_t)f32_to_bf16_bits(o[i]);
      else
        static_cast<float*>(out_col)[oi] = o[i];
    }
  }
}

// SiLU with the hardware exponential and reciprocal.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + __expf(-z));
}

// Gated tail: w * SiLU(z) of token tile W of chunk j into the Gz ring (chain
// wave W, in phase C where it only prefetches); lane l takes token
// 16 W + l / 4, columns 4 (l % 4) .. 4 (l % 4) + 3.
constexpr int kGzLag = 3;         // chunk c computes it for chunk c - 3
template <int W>
__device__ __forceinline__ void gate_z(ScanLds& sm, int j, int lane) {
  const int tok = 16 * W + (lane >> 2), q = lane & 3;
  const uint2 zz = *reinterpret_cast<const uint2*>(&sm.Z[j & 7][tok * kSliceRows + 4 * q]);
  const f32x4_t w = *reinterpret_cast<const f32x4_t*>(&sm.wn[4 * q]);
  const uint32_t zw[2] = {zz.x, zz.y};
  f32x4_t gz;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t zb = (e & 1) ? (zw[e >> 1] >> 16) : (zw[e >> 1] & 0xffffu);
    gz[e] = w[e] * silu_fast(bf16_bits_to_f32(zb));
  }
  *reinterpret_cast<f32x4_t*>(&sm.Gz[j & 7][tok * kSliceRows + 4 * q]) = gz;
}

// One chunk ci of chain wave W: K / Q fragments in `kq` (each reloaded with
// chunk ci + 2 after its last use: K at the end of phase A, Q in phase C),
// T fragments in `t` (reloaded with chunk ci + 1).  The vector-memory path
// of the compute unit is the scarce resource of the loads: spreading them
// over the phases keeps any one phase from waiting for it.
template <int W, bool GATED>
__device__ __forceinline__ void chain_chunk(ScanLds& sm, ChainOps<W>& kq,
                                            TOps<W>& t, const ScanCtx& x,
                                            int ci, int lane) {
  constexpr int nks = ChainOps<W>::nks;
  const int g = lane >> 4, c = lane & 15;
  const int slot = ci % 3;
  // Phase A: X = K S0^T; R; K into the LDS tile.
  bf16x8_t sh[4], sl[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    sh[ks] = ld8(sm.Sh, sw128(c, 32 * ks + 8 * g));
    sl[ks] = ld8(sm.Sl, sw128(c, 32 * ks + 8 * g));
  }
  f32x4_t X = {0.f, 0.f, 0.f, 0.f}, X2 = X;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    X = mfma32(kq.kf[ks], sh[ks], X);
    X2 = mfma32(kq.kf[ks], sl[ks], X2);
  }
  const int rowo = 16 * W + 4 * g;
  const f32x4_t eg = *reinterpret_cast<const f32x4_t*>(&sm.gate[slot][rowo]);
  const f32x4_t bb = *reinterpret_cast<const f32x4_t*>(&sm.gate[slot][2 * kC + rowo]);
  f32x4_t R;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float vv = bf16_bits_to_f32(sm.V[slot][(rowo + i) * kSliceRows + c]);
    R[i] = bb[i] * (vv - eg[i] * (X[i] + X2[i]));
  }
  store_split4p(sm.Rh, sm.Rl, sw64(c, 16 * W + 4 * g), R);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    *reinterpret_cast<bf16x8_t*>(&sm.Kb[sw128k(16 * W + c, 32 * ks + 8 * g)]) = kq.kf[ks];
  load_k<W>(kq, x, ci + 2, lane);
  lds_barrier();
  // Phase B: U = T R; W = diag(e^{G_L - G}) U.  Y = Q S0^T is issued first:
  // its products fill the matrix core while the R reads are in flight.
  bf16x8_t rh[nks], rl[nks];
#pragma unroll
  for (int ks = 0; ks < nks; ++ks) {
    rh[ks] = ld8(sm.Rh, sw64(c, 32 * ks + 8 * g));
    rl[ks] = ld8(sm.Rl, sw64(c, 32 * ks + 8 * g));
  }
  f32x4_t Y = {0.f, 0.f, 0.f, 0.f}, Y2 = Y;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    Y = mfma32(kq.qf[ks], sh[ks], Y);
    Y2 = mfma32(kq.qf[ks], sl[ks], Y2);
  }
  f32x4_t U = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < nks; ++ks) {
    U = mfma32(t.th[ks], rh[ks], U);
    U = mfma32(t.th[ks], rl[ks], U);
    U = mfma32(t.tl[ks], rh[ks], U);
  }
  load_tp<W>(t, x, ci + 1, 0, lane);
  const f32x4_t egl = *reinterpret_cast<const f32x4_t*>(&sm.gate[slot][kC + rowo]);
  store_split4p(sm.Wh, sm.Wl, sw64(c, 16 * W + 4 * g), egl * U);
  store_split4p(sm.Uh, sm.Ul, sw64(c, 16 * W + 4 * g), U);
  sm.Y[W][lane] = Y + Y2;
  lds_barrier();
  // Phase C: the state update runs on the state waves; this wave only
  // prefetches (and for the gated tail prepares w * SiLU(z)).
  load_q<W>(kq, x, ci + 2, lane);
  if constexpr (GATED)
    if (ci >= kGzLag) gate_z<W>(sm, ci - kGzLag, lane);
  lds_barrier();
}

template <int W, bool GATED>
__device__ __forceinline__ void scan_chain(ScanLds& sm, const ScanCtx& x,
                                           int lane) {
  // The chain waves carry the serial part of every chunk: they win issue
  // arbitration against the state wave sharing their SIMD.
  __builtin_amdgcn_s_setprio(2);
  const int nch = x.nch;
  ChainOps<W> a, b;
  TOps<W> t;
  load_kq<W>(a, x, 0, lane);
  load_kq<W>(b, x, 1, lane);
  load_tp<W>(t, x, 0, 0, lane);
  lds_barrier();   // initial state, V and gates of chunks 0 and 1 in LDS
  chain_chunk<W, GATED>(sm, a, t, x, 0, lane);
  int ci = 1;
  for (; ci + 1 < nch; ci += 2) {
    chain_chunk<W, GATED>(sm, b, t, x, ci, lane);
    chain_chunk<W, GATED>(sm, a, t, x, ci + 1, lane);
  }
  if (ci < nch) chain_chunk<W, GATED>(sm, b, t, x, ci, lane);
  if constexpr (GATED) {
    // w * SiLU(z) of the last chunks, before the tail waves finish them.
    for (int j = nch > kGzLag ? nch - kGzLag : 0; j < nch; ++j) gate_z<W>(sm, j, lane);
    lds_barrier();
    lds_barrier();
  }
}

// Read-out of chunk ci on state wave 4 + J (token tile J): O = diag(e^G) Y
// + P U from the LDS Y, U and gates of that chunk.
template <int J>
__device__ __forceinline__ f32x4_t readout(const ScanLds& sm, const TOps<J>& p,
                                           int ci, int lane) {
  const int g = lane >> 4, c = lane & 15;
  const f32x4_t eg = *reinterpret_cast<const f32x4_t*>(&sm.gate[ci % 3][16 * J + 4 * g]);
  f32x4_t O = eg * sm.Y[J][lane];
#pragma unroll
  for (int ks = 0; ks < ChainOps<J>::nks; ++ks) {
    const bf16x8_t uh = ld8(sm.Uh, sw64(c, 32 * ks + 8 * g));
    const bf16x8_t ul = ld8(sm.Ul, sw64(c, 32 * ks + 8 * g));
    O = mfma32(p.th[ks], uh, O);
    O = mfma32(p.th[ks], ul, O);
    O = mfma32(p.tl[ks], uh, O);
  }
  return O;
}

// ------------------------------------------------------ fused gated tail --
// The gated RMSNorm ("Red Lite dev15d -- DeltaNet gated tail + Q4_K output
// projection", Pinned graph semantics steps 2-5) needs, per token and value
// head, the sum of squares of o over all 128 columns, which 8 slice
// workgroups hold 16 columns each.  It runs a few chunks behind the scan:
//  - chunk c, phase A: the state waves put read-out c - 1 in LDS (ring
//    slot (c - 1) % 8, token-major);
//  - chunk c, phase C: the exchange wave (lane t = token t of a chunk)
//    stores this slice's sums of squares of chunk c - 1's tokens into their
//    slots (which the prep kernel set to -1).  On slice 0 it also adds the 8
//    slices' sums of chunk c - 4 that it loaded at chunk c - 1 (re-reading
//    them until none is -1), publishes the total in a ninth slot and puts
//    1 / RMS in LDS, then loads the sums of chunk c - 3; on the other slices
//    it takes 1 / RMS of chunk c - 6 from the total it loaded at chunk c - 1
//    (re-read until it is not -1) and loads the total of chunk c - 5, which
//    slice 0 published a chunk earlier.  One reader of 8 slots per group, 7
//    of one, instead of 8 of 8;
//  - chunk c, phase C: each chain wave puts w * SiLU(z) of its token tile of
//    chunk c - 3 in LDS (z staged with V);
//  - chunk c, phase A: the output wave writes chunk c - 7 (normalised by
//    chunk c - 1's phase C on every slice), o * (1 / RMS) * (w * SiLU(z)).
//    It issues no load, so its stores never hold up a wait.
// Phase C is where the chain waves only prefetch: the exchange's memory
// latency and the SiLU work there hold up no dependent step.
// Sums are written and read with relaxed device-scope atomics, which go to
// the memory side of the caches, one 4-byte value each, so a value read is
// either -1 or the sum.  The slices of a group must run at the same time:
// the kernel is launched cooperatively (all workgroups resident) and each
// workgroup walks its team's groups in the same order.  Slice 0 waits at
// chunk c for sums every slice stored at chunk c - 3; the others wait for a
// total slice 0 stored at chunk c - 2, after its own wait.  No wait is on a
// slice behind the waiter in a cycle, so the waits end; each is also
// bounded.  (With the ring of 8 chunk slots, the read-out of chunk c - 1
// stored at chunk c and the output of chunk c - 7 are 6 slots apart.)
constexpr int kTailLag = 4;       // slice 0 normalises chunk c - 4 at chunk c
constexpr int kTotLag = 6;        // the other slices chunk c - 6
constexpr int kOutLag = 7;        // and every slice writes chunk c - 7

// Polls of one wait (each after a short sleep) before it gives up; a wave
// whose wait gave up writes what it has and no longer waits, so even a
// broken residency guarantee cannot hold the kernel for long.
constexpr int kSpinLimit = 1 << 16;

// What the exchange wave needs of its group and slice.
struct TailLoad {
  float* part;          // the group's first chunk: [9 slots][64 tokens]
  int64_t stride;       // floats between consecutive chunks
  float eps;
  int sl;               // this slice
  bool stuck;           // a wait has run out: later ones do not spin
};

// Where the output wave writes: for token tile J, lane l writes token
// 16 J + l / 4, columns 4 (l % 4) .. 4 (l % 4) + 3 of the slice.
struct TailOut {
  void* out;            // output row of that token of the first chunk, at its
  int64_t row;          //   first column; elements between rows
};

// Slice 0 reads the 8 slices' sums of chunk j; the others its total (v[0]).
__device__ __forceinline__ void load_sums8(const TailLoad& tl, float (&v)[kSlices], int j,
                                           int lane) {
  const float* at = tl.part + j * tl.stride + lane;
  if (tl.sl == 0) {
#pragma unroll
    for (int s8 = 0; s8 < kSlices; ++s8)
      v[s8] = __hip_atomic_load(at + s8 * kC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    v[0] = __hip_atomic_load(at + kSlices * kC, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}
__device__ __forceinline__ bool all_stored(const TailLoad& tl, const float (&v)[kSlices]) {
  bool ok = !(v[0] < 0.f);
  if (tl.sl == 0) {
#pragma unroll
    for (int s8 = 1; s8 < kSlices; ++s8) ok = ok && !(v[s8] < 0.f);
  }
  return __all(ok);
}

// Re-reads chunk j's sums until none is -1 (entered only after a first test
// failed, so that the common case waits for no later memory operation; it
// leaves no load in flight).
__device__ __forceinline__ void await_sums8(TailLoad& tl, float (&v)[kSlices], int j,
                                            int lane) {
  for (int spin = 0; !tl.stuck; ++spin) {
    if (spin == kSpinLimit) {
      tl.stuck = true;
      break;
    }
    __builtin_amdgcn_s_sleep(1);
    load_sums8(tl, v, j, lane);
    if (all_stored(tl, v)) break;
  }
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
}

// The lane's token's sum of squares over all 128 columns: on slice 0 the 8
// slice sums added in slice order, elsewhere the total slice 0 published.
__device__ __forceinline__ float total_of(const TailLoad& tl, const float (&v)[kSlices]) {
  if (tl.sl != 0) return v[0];
  float total = 0.f;
#pragma unroll
  for (int s8 = 0; s8 < kSlices; ++s8) total += v[s8];
  return total;
}
__device__ __forceinline__ float rstd_from(const TailLoad& tl, float total) {
  return __builtin_amdgcn_rsqf(total / (float)kD + tl.eps);
}
// Normalises chunk j (its values loaded into v): slice 0 publishes the
// total first.
__device__ __forceinline__ void normalise(ScanLds& sm, TailLoad& tl, float (&v)[kSlices],
                                          int j, int lane) {
  if (!all_stored(tl, v) && !tl.stuck) await_sums8(tl, v, j, lane);
  const float total = total_of(tl, v);
  if (tl.sl == 0)
    __hip_atomic_store(tl.part + j * tl.stride + kSlices * kC + lane, total, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  sm.rstd[j & 7][lane] = rstd_from(tl, total);
}

// This slice's sum of squares of token `lane` of read-out j (from LDS).
__device__ __forceinline__ float slice_sum(const ScanLds& sm, int j, int lane) {
  const f32x4_t* r = reinterpret_cast<const f32x4_t*>(&sm.Ot[j & 7][lane * kOtLd]);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x4_t x = r[k];
    s += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
  }
  return s;
}

// Exchange wave's step at chunk ci: 1 / RMS of chunk ci - lag into LDS
// (from `v`, loaded one chunk earlier; lag 4 on slice 0, 6 elsewhere), this
// slice's sums of chunk ci - 1, loads for chunk ci - lag + 1 into `v` -- the
// wave's last memory operations, so the next step's wait for them waits for
// nothing else.
__device__ __forceinline__ void tail_step(ScanLds& sm, TailLoad& tl, float (&v)[kSlices],
                                          int ci, int lane) {
  const int lag = tl.sl == 0 ? kTailLag : kTotLag;
  const int jt = ci - lag;
  if (jt >= 0) normalise(sm, tl, v, jt, lane);
  const int js = ci - 1;
  const float mine = js >= 0 ? slice_sum(sm, js, lane) : -1.f;
  __hip_atomic_store(tl.part + (js > 0 ? js : 0) * tl.stride + tl.sl * kC + lane, mine,
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int jl = ci - lag + 1;
  load_sums8(tl, v, jl > 0 ? jl : 0, lane);
}

// The read-out of chunk ci - 1 (state wave 4 + J, lane (g, c): tokens 16 J
// + 4 g + i, column c) into the ring.
template <int J>
__device__ __forceinline__ void keep_readout(ScanLds& sm, f32x4_t o, int ci, int lane) {
  const int g = lane >> 4, c = lane & 15;
  float* r = &sm.Ot[(ci - 1) & 7][(16 * J + 4 * g) * kOtLd + c];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i * kOtLd] = o[i];
}

// Gated output of token tile J of chunk j (see TailOut), tokens below L.
template <int OUT, int J>
__device__ __forceinline__ void finish_out(const ScanLds& sm, const TailOut& to, int j, int L,
                                           int lane) {
  const int tok = 16 * J + (lane >> 2), q = lane & 3;
  const float rs = sm.rstd[j & 7][tok];
  const f32x4_t o = *reinterpret_cast<const f32x4_t*>(&sm.Ot[j & 7][tok * kOtLd + 4 * q]);
  const f32x4_t gz = *reinterpret_cast<const f32x4_t*>(&sm.Gz[j & 7][tok * kSliceRows + 4 * q]);
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = o[e] * rs * gz[e];
  if (tok < L) {
    const int64_t at = ((int64_t)j * kC + tok) * to.row;
    if constexpr (out_is_bf16(OUT)) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(to.out) + at) =
          make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(to.out) + at) =
          make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

// One chunk ci of state wave 4 + J.  Except in the first chunk, the
// read-out of chunk ci - 1 comes first (its U, Y and gates are still in
// LDS, its P fragments in `p`, which is then reloaded with chunk ci): it is
// stored, or for the gated tail kept in LDS (see above).
template <int OUT, int J, bool FIRST>
__device__ __forceinline__ void state_chunk(ScanLds& sm, TOps<J>& p,
                                            f32x4_t (&acc)[2], const ScanCtx& x,
                                            void* out_col, int64_t out_stride,
                                            int ci, int lane) {
  const int g = lane >> 4, c = lane & 15;
  // Phase A: read-out of the previous chunk (a full chunk); scale the state.
  if constexpr (!FIRST) {
    const f32x4_t O = readout<J>(sm, p, ci - 1, lane);
    if constexpr (is_gated(OUT)) {
      keep_readout<J>(sm, O, ci, lane);
    } else {
      store_out<OUT>(out_col, out_stride, O, ci - 1, kC, 16 * J + 4 * g);
    }
    load_tp<J>(p, x, ci, 1, lane);
  }
  const float eL = sm.gate[ci % 3][kC - 1];
  acc[0] *= eL;
  acc[1] *= eL;
  lds_barrier();
  // Phase B: the chain computes U and W.
  lds_barrier();
  // Phase C: S^T += K^T W on dimension tiles 2J, 2J + 1; S as hi / lo.
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const bf16x8_t wh = ld8(sm.Wh, sw64(c, 32 * ks + 8 * g));
    const bf16x8_t wl = ld8(sm.Wl, sw64(c, 32 * ks + 8 * g));
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
      const bf16x8_t kt = kt_frag(sm.Kb, 2 * J + dl, ks, lane);
      acc[dl] = mfma32(kt, wh, acc[dl]);
      acc[dl] = mfma32(kt, wl, acc[dl]);
    }
  }
#pragma unroll
  for (int dl = 0; dl < 2; ++dl)
    store_split4p(sm.Sh, sm.Sl, sw128(c, 16 * (2 * J + dl) + 4 * g), acc[dl]);
  lds_barrier();
}

template <int OUT, int J>
__device__ __forceinline__ void scan_state(ScanLds& sm, const PrefillParams& p,
                                           const Maps& m, const ScanCtx& x,
                                           int lane, int grp, int q0, int h, int sl,
                                           int v0, int64_t t_beg, int64_t srow) {
  const int g = lane >> 4, c = lane & 15;
  const int64_t row = (int64_t)p.h_v * kD;
  const int64_t ocol = (t_beg * p.h_v + h) * kD + v0 + c;
  void* out_col = out_is_bf16(OUT) ? static_cast<void*>(static_cast<uint16_t*>(p.out) + ocol)
                                   : static_cast<void*>(static_cast<float*>(p.out) + ocol);
  f32x4_t acc[2];
#pragma unroll
  for (int dl = 0; dl < 2; ++dl) {
    const int col = 16 * (2 * J + dl) + 4 * g;
    if (p.s0) {
      const float4 v = *reinterpret_cast<const float4*>(p.s0 + srow + col);
      acc[dl] = f32x4_t{v.x, v.y, v.z, v.w};
    } else {
      acc[dl] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    store_split4p(sm.Sh, sm.Sl, sw128(c, col), acc[dl]);
  }
  const int nch = x.nch;
  TOps<J> pf;
  load_tp<J>(pf, x, 0, 1, lane);
  lds_barrier();
  state_chunk<OUT, J, true>(sm, pf, acc, x, out_col, row, 0, lane);
  for (int ci = 1; ci < nch; ++ci)
    state_chunk<OUT, J, false>(sm, pf, acc, x, out_col, row, ci, lane);
  // Read-out of the last chunk (L tokens).
  const int64_t rem = x.len - (int64_t)(nch - 1) * kC;
  const int L = (int)(rem < kC ? rem : kC);
  const f32x4_t O = readout<J>(sm, pf, nch - 1, lane);
  if constexpr (is_gated(OUT)) {
    // After the exchange wave's last normalisers: the remaining outputs.
    keep_readout<J>(sm, O, nch, lane);
    lds_barrier();
    lds_barrier();
  } else {
    store_out<OUT>(out_col, row, O, nch - 1, L, 16 * J + 4 * g);
  }
  if (p.sF) {
#pragma unroll
    for (int dl = 0; dl < 2; ++dl) {
      const int col = 16 * (2 * J + dl) + 4 * g;
      *reinterpret_cast<float4*>(p.sF + srow + col) =
          make_float4(acc[dl][0], acc[dl][1], acc[dl][2], acc[dl][3]);
    }
  }
}

// Direct-to-LDS loads of one chunk's V slice (rows past the end of a short
// chunk repeat its last token: they meet b = 0 and are never stored) and
// gate record into ring slot ci % 3 (three loads), and for the gated tail
// its z slice into slot ci % 8 (two more).
template <bool GATED>
constexpr int stage_loads() { return GATED ? 5 : 3; }
template <bool GATED>
__device__ __forceinline__ void stage_chunk(ScanLds& sm, const PrefillParams& p,
                                            const ScanCtx& x, int64_t t_beg,
                                            int h, int v0, int ci, int lane) {
  const int zslot = ci & 7;
  // The ring slot of chunk ci even past the last chunk (then the source is
  // the last chunk again): that slot's previous chunk is no longer read.
  const int slot = ci % 3;
  ci = clamp_chunk(x, ci);
  const int64_t rem = x.len - (int64_t)ci * kC;
  const int L = (int)(rem < kC ? rem : kC);
  const uint16_t* vg = static_cast<const uint16_t*>(p.v);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int tok = min(32 * i + (lane >> 1), L - 1);
    dma16(vg + ((t_beg + (int64_t)ci * kC + tok) * p.h_v + h) * kD + v0 + 8 * (lane & 1),
          &sm.V[slot][32 * i * kSliceRows]);
  }
  // The 768-byte gate record is 48 lanes' worth: lane l's 16 bytes land at
  // the slot base + 16 l, so lanes past 47 must not load.
  if (lane < 48) dma16(x.gate0 + ci * x.gate_stride + 4 * lane, &sm.gate[slot][0]);
  if constexpr (GATED) {
    const uint16_t* zg = static_cast<const uint16_t*>(p.z);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tok = min(32 * i + (lane >> 1), L - 1);
      dma16(zg + ((t_beg + (int64_t)ci * kC + tok) * p.h_v + h) * kD + v0 + 8 * (lane & 1),
            &sm.Z[zslot][32 * i * kSliceRows]);
    }
  }
}

// Loader wave: chunks 0 and 1 are staged before the first barrier, then
// chunk ci + 2 during phase B of chunk ci; before the last barrier of chunk
// ci it waits for chunk ci + 1's loads (issued one chunk earlier), leaving
// chunk ci + 2's in flight.  (It writes LDS only through these loads: any
// LDS access of its own would have to wait for all of them.)
template <bool GATED>
__device__ __forceinline__ void scan_loader(ScanLds& sm, const PrefillParams& p,
                                            const ScanCtx& x, int64_t t_beg, int h,
                                            int v0, int lane) {
  stage_chunk<GATED>(sm, p, x, t_beg, h, v0, 0, lane);
  stage_chunk<GATED>(sm, p, x, t_beg, h, v0, 1, lane);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  raw_barrier();
  for (int ci = 0; ci < x.nch; ++ci) {
    raw_barrier();
    stage_chunk<GATED>(sm, p, x, t_beg, h, v0, ci + 2, lane);
    raw_barrier();
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(stage_loads<GATED>()));
    raw_barrier();
  }
  // No load may still be writing the workgroup's LDS when it is released.
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  if constexpr (GATED) {
    raw_barrier();
    raw_barrier();
  }
}

// What the exchange wave needs of its group and slice.
__device__ __forceinline__ TailLoad tail_ctx(const PrefillParams& p, const Maps& m, int h,
                                             int q0, int sl) {
  TailLoad tl{};
  tl.part = m.part + ((int64_t)q0 * p.h_v + h) * kSlots * kC;
  tl.stride = (int64_t)p.h_v * kSlots * kC;
  tl.sl = sl;
  tl.eps = p.eps;
  return tl;
}

// Exchange wave (gated tail only; otherwise it only meets the barriers).
template <int OUT>
__device__ __forceinline__ void scan_exchange(ScanLds& sm, const PrefillParams& p,
                                              const Maps& m, const ScanCtx& x, int h,
                                              int q0, int sl, int lane) {
  constexpr bool GATED = is_gated(OUT);
  TailLoad tl{};
  float v[kSlices];
  if constexpr (GATED) {
    tl = tail_ctx(p, m, h, q0, sl);
    if (lane < kSliceRows) sm.wn[lane] = p.w[sl * kSliceRows + lane];
  }
  lds_barrier();
  const int nch = x.nch;
  for (int ci = 0; ci < nch; ++ci) {
    lds_barrier();
    lds_barrier();
    if constexpr (GATED) tail_step(sm, tl, v, ci, lane);
    lds_barrier();
  }
  if constexpr (GATED) {
    // The state waves have put the last read-out in LDS: publish its sums,
    // then normalise the chunks the loop has not (the last 4 on slice 0,
    // the last 6 elsewhere).
    lds_barrier();
    __hip_atomic_store(tl.part + (nch - 1) * tl.stride + sl * kC + lane,
                       slice_sum(sm, nch - 1, lane), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    const int lag = sl == 0 ? kTailLag : kTotLag;
    for (int j = nch > lag ? nch - lag : 0; j < nch; ++j) {
      load_sums8(tl, v, j, lane);
      normalise(sm, tl, v, j, lane);
    }
    lds_barrier();
  }
}

// Output wave (gated tail only; otherwise it only meets the barriers): in
// phase A of chunk ci it writes chunk ci - 5.  It issues no load, so its
// stores never hold up a wait.
template <int OUT>
__device__ __forceinline__ void finish_chunk(const ScanLds& sm, const TailOut& to, int j,
                                             int L, int lane) {
  finish_out<OUT, 0>(sm, to, j, L, lane);
  finish_out<OUT, 1>(sm, to, j, L, lane);
  finish_out<OUT, 2>(sm, to, j, L, lane);
  finish_out<OUT, 3>(sm, to, j, L, lane);
}
template <int OUT>
__device__ __forceinline__ void scan_output(ScanLds& sm, const PrefillParams& p,
                                            const ScanCtx& x, int h, int v0, int64_t t_beg,
                                            int lane) {
  constexpr bool GATED = is_gated(OUT);
  TailOut to{};
  if constexpr (GATED) {
    const int q = lane & 3;
    const int64_t col = (t_beg * p.h_v + h) * kD + v0 + 4 * q;
    to.out = out_is_bf16(OUT) ? static_cast<void*>(static_cast<uint16_t*>(p.out) + col)
                              : static_cast<void*>(static_cast<float*>(p.out) + col);
    to.row = (int64_t)p.h_v * kD;
  }
  lds_barrier();
  const int nch = x.nch;
  for (int ci = 0; ci < nch; ++ci) {
    if constexpr (GATED)
      if (ci >= kOutLag) finish_chunk<OUT>(sm, to, ci - kOutLag, kC, lane);
    lds_barrier();
    lds_barrier();
    lds_barrier();
  }
  if constexpr (GATED) {
    lds_barrier();
    lds_barrier();
    const int64_t rem = x.len - (int64_t)(nch - 1) * kC;
    for (int j = nch > kOutLag ? nch - kOutLag : 0; j < nch; ++j)
      finish_chunk<OUT>(sm, to, j, j == nch - 1 ? (int)(rem < kC ? rem : kC) : kC, lane);
  }
}

// One work item: a (sequence, value head) group as one slice sees it.
struct Group {
  ScanCtx x;
  int64_t t_beg, srow;
  int grp, h, q0;
};

__device__ __forceinline__ Group make_group(const PrefillParams& p, const Maps& m,
                                            int grp, int v0, int c) {
  Group G;
  G.grp = grp;
  const int n = m.seq_order[grp / p.h_v];
  G.h = grp - (grp / p.h_v) * p.h_v;
  const int hk = G.h / p.group;
  int64_t t_end;
  seq_range(m, n, G.t_beg, t_end);
  G.q0 = m.prefix[n];
  G.x.nch = m.prefix[n + 1] - G.q0;
  G.x.len = t_end - G.t_beg;
  G.x.kq0 = m.kqf + ((int64_t)G.q0 * p.h_k + hk) * kKqU4;
  G.x.kq_stride = (int64_t)p.h_k * kKqU4;
  G.x.rec0 = m.rec + ((int64_t)G.q0 * p.h_v + G.h) * kRecU4;
  G.x.rec_stride = (int64_t)p.h_v * kRecU4;
  G.x.gate0 = m.gate + ((int64_t)G.q0 * p.h_v + G.h) * 3 * kC;
  G.x.gate_stride = (int64_t)p.h_v * 3 * kC;
  G.srow = (((int64_t)n * p.h_v + G.h) * kD + v0 + c) * kD;
  return G;
}

// Runs `body` for each group of the team; every wave of the workgroup walks
// the same groups and meets a barrier before each (the previous group's
// last reads of the LDS ring are then done).
template <bool LOADER, typename F>
__device__ __forceinline__ void for_groups(const PrefillParams& p, const Maps& m,
                                           int team, int teams, int v0, int c,
                                           F&& body) {
  for (int grp = team; grp < p.N * p.h_v; grp += teams) {
    if constexpr (LOADER) raw_barrier(); else lds_barrier();
    body(make_group(p, m, grp, v0, c));
  }
}

// Empty sequence: the final state is the initial one (state wave 4 + J).
template <int J>
__device__ __forceinline__ void copy_state(const PrefillParams& p, int64_t srow, int g) {
  if (!p.sF) return;
#pragma unroll
  for (int dl = 0; dl < 2; ++dl) {
    const int col = 16 * (2 * J + dl) + 4 * g;
    const float4 v = p.s0 ? *reinterpret_cast<const float4*>(p.s0 + srow + col)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(p.sF + srow + col) = v;
  }
}

template <int OUT, int J>
__device__ __forceinline__ void state_groups(ScanLds& sm, const PrefillParams& p,
                                             const Maps& m, int team, int teams,
                                             int sl, int v0, int lane) {
  const int g = lane >> 4, c = lane & 15;
  for_groups<false>(p, m, team, teams, v0, c, [&](const Group& G) {
    if (G.x.nch == 0)
      copy_state<J>(p, G.srow, g);
    else
      scan_state<OUT, J>(sm, p, m, G.x, lane, G.grp, G.q0, G.h, sl, v0, G.t_beg, G.srow);
  });
}

template <int OUT>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(PrefillParams p,
                                                            Maps m) {
  __shared__ ScanLds sm;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15;
  const int b = blockIdx.x;
  const int nb = gridDim.x;
  const bool xcd = (nb & 63) == 0;
  // Blocks are dealt to the 8 XCDs round-robin (XCD b % 8).  A team's 8
  // slices sit on one XCD, and consecutive teams -- the value heads that
  // share a key head, whose groups are adjacent -- on the same XCD, so that
  // the second reads that key head's K / Q fragments from its L2.
  const int team = xcd ? (nb >> 6) * (b & 7) + (b >> 6) : b >> 3;
  const int sl = xcd ? (b >> 3) & 7 : b & 7;
  const int teams = nb >> 3;
  const int v0 = sl * kSliceRows;
  switch (w) {
#define GDN_CHAIN(W)                                                        \
  case W:                                                                   \
    for_groups<false>(p, m, team, teams, v0, c, [&](const Group& G) {       \
      if (G.x.nch > 0) {                                                    \
        scan_chain<W, is_gated(OUT)>(sm, G.x, lane);                        \
      }                                                                     \
    });                                                                     \
    break;
    GDN_CHAIN(0)
    GDN_CHAIN(1)
    GDN_CHAIN(2)
    GDN_CHAIN(3)
#undef GDN_CHAIN
    case 4: state_groups<OUT, 0>(sm, p, m, team, teams, sl, v0, lane); break;
    case 5: state_groups<OUT, 1>(sm, p, m, team, teams, sl, v0, lane); break;
    case 6: state_groups<OUT, 2>(sm, p, m, team, teams, sl, v0, lane); break;
    case 7: state_groups<OUT, 3>(sm, p, m, team, teams, sl, v0, lane); break;
    case 8:
      for_groups<true>(p, m, team, teams, v0, c, [&](const Group& G) {
        if (G.x.nch > 0) scan_loader<is_gated(OUT)>(sm, p, G.x, G.t_beg, G.h, v0, lane);
      });
      break;
    case 9:
      for_groups<false>(p, m, team, teams, v0, c, [&](const Group& G) {
        if (G.x.nch > 0) scan_exchange<OUT>(sm, p, m, G.x, G.h, G.q0, sl, lane);
      });
      break;
    default:
      for_groups<false>(p, m, team, teams, v0, c, [&](const Group& G) {
        if (G.x.nch > 0) scan_output<OUT>(sm, p, G.x, G.h, v0, G.t_beg, lane);
      });
      break;
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t prefix, seq_beg, seq_end, seq_order, chunk_seq, rec, kqf, gate, part,
      total;
  int32_t QB;
};

WsLayout ws_layout(int64_t T, int32_t N, int32_t h_k, int32_t h_v,
                   int32_t d_v, bool tail) {
  WsLayout l;
  l.QB = (int32_t)(T / kC + N);
  size_t off = 0;
  l.prefix = off;    off += align256(sizeof(int32_t) * (N + 1));
  l.seq_beg = off;   off += align256(sizeof(int32_t) * N);
  l.seq_end = off;   off += align256(sizeof(int32_t) * N);
  l.seq_order = off; off += align256(sizeof(int32_t) * N);
  l.chunk_seq = off; off += align256(sizeof(int32_t) * (size_t)l.QB);
  l.rec = off;       off += align256(sizeof(uint4) * (size_t)l.QB * h_v * kRecU4);
  l.kqf = off;       off += align256(sizeof(uint4) * (size_t)l.QB * h_k * kKqU4);
  l.gate = off;      off += align256(sizeof(float) * (size_t)l.QB * h_v * 3 * kC);
  l.part = off;      off += tail ? align256(sizeof(float) * (size_t)l.QB * h_v * kSlots * kC) : 0;
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
  m.seq_beg = reinterpret_cast<int32_t*>(base + l.seq_beg);
  m.seq_end = reinterpret_cast<int32_t*>(base + l.seq_end);
  m.seq_order = reinterpret_cast<int32_t*>(base + l.seq_order);
  m.chunk_seq = reinterpret_cast<int32_t*>(base + l.chunk_seq);
  m.rec = reinterpret_cast<uint4*>(base + l.rec);
  m.kqf = reinterpret_cast<uint4*>(base + l.kqf);
  m.gate = reinterpret_cast<float*>(base + l.gate);
  m.part = p.tail ? reinterpret_cast<float*>(base + l.part) : nullptr;
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
  // One team of 8 blocks per group, the grid a multiple of 64 blocks (see
  // scan_kernel).
  const int64_t groups = (int64_t)p.N * p.h_v;
  int64_t blocks = (groups + 7) / 8 * 64;
  if (blocks == 0) return hipSuccess;
  const int mode = p.tail ? (p.out_bf16 ? kOutGatedBf16 : kOutGatedF32)
                          : (p.out_bf16 ? kOutBf16 : kOutF32);
  const void* fn = mode == kOutGatedBf16 ? reinterpret_cast<const void*>(&scan_kernel<kOutGatedBf16>)
                 : mode == kOutGatedF32  ? reinterpret_cast<const void*>(&scan_kernel<kOutGatedF32>)
                 : mode == kOutBf16      ? reinterpret_cast<const void*>(&scan_kernel<kOutBf16>)
                                         : reinterpret_cast<const void*>(&scan_kernel<kOutF32>);
  if (is_gated(mode)) {
    // The slices of a group wait for each other: the whole grid must be
    // resident, so it is capped at what the device holds at once (a
    // multiple of 64 blocks when it holds 64 or more) and launched
    // cooperatively, which fails rather than run a grid that does not fit.
    int dev = 0, cus = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
      return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kScanThreads, 0)) !=
        hipSuccess)
      return e;
    const int64_t resident = (int64_t)cus * per_cu;
    const int64_t cap = resident >= 64 ? resident / 64 * 64 : resident / 8 * 8;
    if (cap < 8) return hipErrorCooperativeLaunchTooLarge;
    if (blocks > cap) blocks = cap;
    void* args[] = {const_cast<PrefillParams*>(&p), &m};
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)blocks), dim3(kScanThreads), args, 0,
                                      stream);
  }
  if (mode == kOutBf16)
    hipLaunchKernelGGL(scan_kernel<kOutBf16>, dim3((unsigned)blocks), dim3(kScanThreads), 0,
                       stream, p, m);
  else
    hipLaunchKernelGGL(scan_kernel<kOutF32>, dim3((unsigned)blocks), dim3(kScanThreads), 0,
                       stream, p, m);
  return hipGetLastError();
}

}  // namespace gdn
