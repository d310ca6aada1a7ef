// proj.hip -- the output projection that follows the gated tail:
// y[m, :] = W x[m, :] for every token m, W being [N out rows, K] in dense
// bf16, in packed Q4_K blocks that the kernels decode themselves, or in the
// low-precision FP8 / MXFP4 codes with activations quantized on the GPU (see
// the low-precision section further down).
//
// "Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection",
// Pinned graph semantics step 6 (the flattened 4096-value tail output
// multiplied by ssm_out, giving the 2048-value hidden vector) and "Q4_K
// implementation": a block packs 256 consecutive values of one weight row in
// 144 bytes -- fp16 d, fp16 dmin, 12 bytes holding eight six-bit sub-block
// scales and eight six-bit sub-block mins, then 128 bytes of four-bit
// quants; a value is d * scale_j * q - dmin * min_j for its 32-value
// sub-block j.  Bit order (the published GGUF layout): scale/min j < 4 are
// the low six bits of bytes j and j + 4; for j >= 4 the low four bits are
// the low (scale) and high (min) nibbles of byte j + 4 and the top two bits
// are the spare top bits of bytes j - 4 (scale) and j (min).  Quant byte l
// of the 32-byte run p carries value l of sub-block 2p in its low nibble and
// value l of sub-block 2p + 1 in its high nibble.
//
// Tile kernel (more than 8 tokens): a workgroup of 4 waves computes a tile
// of BN out rows x BM tokens with v_mfma_f32_16x16x32_bf16, K advancing 64
// values per step through LDS.  Operands that bf16 does not hold exactly are
// split into bf16 parts (RNE of the value, then RNE of each remainder): the
// decoded Q4_K weight, which the loader computes as one fp32 fma of exact
// terms and splits on its way into LDS (2 parts, residual 2^-18, against
// bf16 activations; 3 parts against fp32 ones), and fp32 activations (3
// parts, residual 2^-27).  Accumulation is fp32.
// Matrix-vector kernel (up to 8 tokens): one wave per out row, fp32
// decoding and fp32 fma, the weight row streamed once.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_proj.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kQBlock = 256;       // values per Q4_K block
constexpr int kQBytes = 144;       // bytes per Q4_K block
constexpr int kBK = 64;            // K values per tile step
constexpr int kGemvMaxRows = 8;

// LDS tiles hold rows of 64 bf16 (eight 16-byte granules); granule q of row
// r sits at granule q ^ (r & 7), so the 8 lanes of a 128-bit read that share
// a granule index but sit on 8 consecutive rows hit 8 distinct bank groups.
__device__ __forceinline__ int sw(int r, int c) {
  return r * kBK + ((((c >> 3) ^ (r & 7)) << 3) | (c & 7));
}

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float half_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Splits 8 fp32 values u into P bf16 granules: part 0 = RNE(u), part i =
// RNE of what parts 0 .. i-1 leave (each remainder is exact in fp32).  Two
// parts leave at most 2^-18 |u|, three leave at most 2^-27 |u|.
template <int P>
__device__ __forceinline__ void split8(const float* u, u32x4_t* parts) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = u[2 * i], b = u[2 * i + 1];
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const uint32_t h = pack_bf16x2(a, b);
      parts[k][i] = h;
      if (k + 1 < P) {
        a -= __uint_as_float(h << 16);
        b -= __uint_as_float(h & 0xffff0000u);
      }
    }
  }
}

// Byte i (0..11) of the 12 scale/min bytes, held in three words.
__device__ __forceinline__ uint32_t sbyte(uint32_t s0, uint32_t s1,
                                          uint32_t s2, int i) {
  const uint32_t w = i < 4 ? s0 : (i < 8 ? s1 : s2);
  return (w >> (8 * (i & 3))) & 0xffu;
}

// Six-bit scale and min of sub-block j.
__device__ __forceinline__ void scale_min(uint32_t s0, uint32_t s1,
                                          uint32_t s2, int j, uint32_t& sc,
                                          uint32_t& mn) {
  if (j < 4) {
    sc = sbyte(s0, s1, s2, j) & 63u;
    mn = sbyte(s0, s1, s2, j + 4) & 63u;
  } else {
    const uint32_t lowb = sbyte(s0, s1, s2, j + 4);
    sc = (lowb & 15u) | ((sbyte(s0, s1, s2, j - 4) >> 6) << 4);
    mn = (lowb >> 4) | ((sbyte(s0, s1, s2, j) >> 6) << 4);
  }
}

// The two sub-blocks (2p and 2p + 1) of a 64-value step: multipliers of q
// and the subtracted offsets, both exact in fp32.
struct SubScales {
  float dsc0, dmm0, dsc1, dmm1;
};

__device__ __forceinline__ SubScales sub_scales(u32x4_t hdr, int p) {
  const float d = half_to_f32(hdr[0] & 0xffffu);
  const float dmin = half_to_f32(hdr[0] >> 16);
  uint32_t sc0, mn0, sc1, mn1;
  scale_min(hdr[1], hdr[2], hdr[3], 2 * p, sc0, mn0);
  scale_min(hdr[1], hdr[2], hdr[3], 2 * p + 1, sc1, mn1);
  return SubScales{d * (float)sc0, dmin * (float)mn0, d * (float)sc1,
                   dmin * (float)mn1};
}

// ------------------------------------------------------------ tile kernel --
// XP, WP: bf16 parts of x and of W in LDS (1 = exact in bf16).  The kernel
// keeps every product of parts (a, b) with a + b < max(XP, WP): bf16 x with
// a Q4_K weight uses 2 weight parts (hi*hi + hi*lo); fp32 x uses 3 parts, and
// 3 weight parts when the weight is Q4_K (6 products, residual ~2^-26).
template <int WF, bool XB, int BM, int BN>
struct TileCfg {
  static constexpr int kXP = XB ? 1 : 3;
  static constexpr int kWP = WF == kFmtBf16 ? 1 : (XB ? 2 : 3);
  static constexpr int kOrder = (kXP > kWP ? kXP : kWP) - 1;
  static constexpr int kTM = BM / 32;          // 16-token tiles per wave
  static constexpr int kTN = BN / 32;          // 16-row tiles per wave
  static constexpr int kAG = BM * 8 / 256;     // x granules per thread
  static constexpr int kBG = BN * 8 / 256;     // dense W granules per thread
  static constexpr int kTPR = 256 / BN;        // Q4_K: threads per W row
  static constexpr int kQB = 32 / kTPR;        // Q4_K: quant bytes per thread
  static_assert(BM % 32 == 0 && BN % 64 == 0 && BN <= 256, "tile shape");
};

// Registers carrying one K-step of global data to its LDS store.
template <int WF, bool XB, int BM, int BN>
struct Stage {
  using C = TileCfg<WF, XB, BM, BN>;
  u32x4_t xa[C::kAG][XB ? 1 : 2];              // bf16: 1 granule; f32: 2
  u32x4_t wb[WF == kFmtQ4K ? 1 : C::kBG];        // dense W granules / header
  u32x4_t wq;                                  // Q4_K quant bytes (kQB)
};

template <int WF, bool XB, int BM, int BN>
__device__ __forceinline__ void load_stage(const ProjParams& p, int64_t m0,
                                           int n0, int k0,
                                           Stage<WF, XB, BM, BN>& st) {
  using C = TileCfg<WF, XB, BM, BN>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::kAG; ++i) {
    const int G = tid + 256 * i;
    const int64_t row = min(m0 + (G >> 3), p.M - 1);
    const int col = k0 + 8 * (G & 7);
    if constexpr (XB) {
      st.xa[i][0] = *reinterpret_cast<const u32x4_t*>(
          static_cast<const uint16_t*>(p.x) + row * p.K + col);
    } else {
      const float* src = static_cast<const float*>(p.x) + row * p.K + col;
      st.xa[i][0] = *reinterpret_cast<const u32x4_t*>(src);
      st.xa[i][1] = *reinterpret_cast<const u32x4_t*>(src + 4);
    }
  }
  if constexpr (WF == kFmtBf16) {
#pragma unroll
    for (int i = 0; i < C::kBG; ++i) {
      const int G = tid + 256 * i;
      const int64_t row = min(n0 + (G >> 3), p.N - 1);
      st.wb[i] = *reinterpret_cast<const u32x4_t*>(
          static_cast<const uint16_t*>(p.w) + row * p.K + k0 + 8 * (G & 7));
    }
  } else {
    const int r = tid / C::kTPR, part = tid % C::kTPR;
    const int64_t row = min(n0 + r, p.N - 1);
    const uint8_t* blk = static_cast<const uint8_t*>(p.w) +
                         row * (int64_t)(p.K / kQBlock) * kQBytes +
                         (int64_t)(k0 / kQBlock) * kQBytes;
    st.wb[0] = *reinterpret_cast<const u32x4_t*>(blk);
    const uint8_t* qs = blk + 16 + 32 * ((k0 / kBK) & 3) + part * C::kQB;
    if constexpr (C::kQB == 16) {
      st.wq = *reinterpret_cast<const u32x4_t*>(qs);
    } else {
      const u32x2_t v = *reinterpret_cast<const u32x2_t*>(qs);
      st.wq = u32x4_t{v[0], v[1], 0u, 0u};
    }
  }
}

// Decodes 4 quant bytes (one word) of the step: low nibbles -> sub-block 2p
// values, high nibbles -> sub-block 2p + 1 values (fp32, one rounding).
__device__ __forceinline__ void decode_word(uint32_t w, const SubScales& s,
                                            float* v0, float* v1) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const uint32_t byte = (w >> (8 * b)) & 0xffu;
    v0[b] = fmaf(s.dsc0, (float)(byte & 15u), -s.dmm0);
    v1[b] = fmaf(s.dsc1, (float)(byte >> 4), -s.dmm1);
  }
}

template <int WF, bool XB, int BM, int BN>
__device__ __forceinline__ void store_stage(uint16_t* sA, uint16_t* sB,
                                            int k0,
                                            const Stage<WF, XB, BM, BN>& st) {
  using C = TileCfg<WF, XB, BM, BN>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::kAG; ++i) {
    const int G = tid + 256 * i;
    const int off = sw(G >> 3, 8 * (G & 7));
    if constexpr (XB) {
      *reinterpret_cast<u32x4_t*>(sA + off) = st.xa[i][0];
    } else {
      float u[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u[j] = __uint_as_float(st.xa[i][0][j]);
        u[4 + j] = __uint_as_float(st.xa[i][1][j]);
      }
      u32x4_t parts[C::kXP];
      split8<C::kXP>(u, parts);
#pragma unroll
      for (int k = 0; k < C::kXP; ++k)
        *reinterpret_cast<u32x4_t*>(sA + k * BM * kBK + off) = parts[k];
    }
  }
  if constexpr (WF == kFmtBf16) {
#pragma unroll
    for (int i = 0; i < C::kBG; ++i) {
      const int G = tid + 256 * i;
      *reinterpret_cast<u32x4_t*>(sB + sw(G >> 3, 8 * (G & 7))) = st.wb[i];
    }
  } else {
    const int r = tid / C::kTPR, part = tid % C::kTPR;
    const SubScales s = sub_scales(st.wb[0], (k0 / kBK) & 3);
    constexpr int kWords = C::kQB / 4;
#pragma unroll
    for (int h = 0; h < kWords / 2; ++h) {
      // 8 quant bytes -> 8 values of each sub-block = one granule each.
      float v0[8], v1[8];
      decode_word(st.wq[2 * h], s, v0, v1);
      decode_word(st.wq[2 * h + 1], s, v0 + 4, v1 + 4);
      u32x4_t p0[C::kWP], p1[C::kWP];
      split8<C::kWP>(v0, p0);
      split8<C::kWP>(v1, p1);
      const int c0 = part * C::kQB + 8 * h;
#pragma unroll
      for (int k = 0; k < C::kWP; ++k) {
        *reinterpret_cast<u32x4_t*>(sB + k * BN * kBK + sw(r, c0)) = p0[k];
        *reinterpret_cast<u32x4_t*>(sB + k * BN * kBK + sw(r, 32 + c0)) = p1[k];
      }
    }
  }
}

// Matrix work of one K-step held in LDS buffer (sA, sB).
template <int WF, bool XB, int BM, int BN>
__device__ __forceinline__ void compute_stage(
    const uint16_t* sA, const uint16_t* sB, int wm, int wn, int g, int c,
    f32x4_t (&acc)[TileCfg<WF, XB, BM, BN>::kTM][TileCfg<WF, XB, BM, BN>::kTN]) {
  using C = TileCfg<WF, XB, BM, BN>;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    bf16x8_t xf[C::kXP][C::kTM], wf[C::kWP][C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
      const int off = sw(wm * (BM / 2) + 16 * i + c, 32 * kc + 8 * g);
#pragma unroll
      for (int k = 0; k < C::kXP; ++k)
        xf[k][i] = *reinterpret_cast<const bf16x8_t*>(sA + k * BM * kBK + off);
    }
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
      const int off = sw(wn * (BN / 2) + 16 * j + c, 32 * kc + 8 * g);
#pragma unroll
      for (int k = 0; k < C::kWP; ++k)
        wf[k][j] = *reinterpret_cast<const bf16x8_t*>(sB + k * BN * kBK + off);
    }
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
      for (int j = 0; j < C::kTN; ++j)
#pragma unroll
        for (int a = 0; a < C::kXP; ++a)
#pragma unroll
          for (int w = 0; w < C::kWP; ++w)
            if (a + w <= C::kOrder)
              // D[n][m]: W rows on the A side, tokens on the B side.
              acc[i][j] = mfma32(wf[w][j], xf[a][i], acc[i][j]);
  }
}

template <int WF, bool XB, bool OB, int BM, int BN>
__global__ __launch_bounds__(256) void proj_tile_kernel(ProjParams p) {
  using C = TileCfg<WF, XB, BM, BN>;
  // Two LDS buffers when both fit in 64 KiB (keeping two workgroups per
  // CU); otherwise one buffer and two barriers per step.
  constexpr int kA = C::kXP * BM * kBK, kB = C::kWP * BN * kBK;
  constexpr bool kDB = 2 * (kA + kB) * 2 <= 64 * 1024;
  __shared__ __align__(16) uint16_t smem[(kDB ? 2 : 1) * (kA + kB)];
  uint16_t* const sA0 = smem;
  uint16_t* const sB0 = smem + kA;
  uint16_t* const sA1 = smem + (kDB ? kA + kB : 0);
  uint16_t* const sB1 = smem + (kDB ? 2 * kA + kB : kA);

  // Tile order: dispatch places block b on XCD b % 8, so the remap gives
  // each XCD a contiguous run of ids.  Ids run over (K range, group of 8
  // token panels, row panel, token panel in the group): the workgroups an
  // XCD holds at once cover an 8 x 8 block of tiles, whose token and weight
  // panels its L2 shares.
  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int lid = (nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int split = lid / tiles, t = lid % tiles;
  constexpr int kGroup = 8;
  const int grp = t / (kGroup * tiles_n), in = t % (kGroup * tiles_n);
  const int gm = min(kGroup, tiles_m - grp * kGroup);   // panels in group
  const int64_t m0 = (int64_t)(grp * kGroup + in % gm) * BM;
  const int n0 = (in / gm) * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4_t acc[C::kTM][C::kTN];
#pragma unroll
  for (int i = 0; i < C::kTM; ++i)
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Two buffers: while step ks is multiplied out of one LDS buffer, step ks+1
  // (loaded two steps earlier) is written to the other and the loads of
  // step ks+2 are in flight, so each load has two steps of matrix work to
  // land.  One barrier per step.  Loads past the range end re-read its last
  // step (clamped, never used) so that no load sits in a branch.
  const int steps = p.K / kBK / p.splits;
  const int ks0 = split * steps, last = ks0 + steps - 1;
  if constexpr (!kDB) {
    // Single buffer: the next step's loads fly during this step's work.
    Stage<WF, XB, BM, BN> st;
    load_stage<WF, XB, BM, BN>(p, m0, n0, ks0 * kBK, st);
    for (int ks = ks0; ks <= last; ++ks) {
      if (ks > ks0) __syncthreads();
      store_stage<WF, XB, BM, BN>(sA0, sB0, ks * kBK, st);
      __syncthreads();
      load_stage<WF, XB, BM, BN>(p, m0, n0, min(ks + 1, last) * kBK, st);
      compute_stage<WF, XB, BM, BN>(sA0, sB0, wm, wn, g, c, acc);
    }
  } else {
  Stage<WF, XB, BM, BN> r0, r1;
  load_stage<WF, XB, BM, BN>(p, m0, n0, ks0 * kBK, r0);
  load_stage<WF, XB, BM, BN>(p, m0, n0, min(ks0 + 1, last) * kBK, r1);
  store_stage<WF, XB, BM, BN>(sA0, sB0, ks0 * kBK, r0);
  __syncthreads();
  load_stage<WF, XB, BM, BN>(p, m0, n0, min(ks0 + 2, last) * kBK, r0);
  for (int ks = ks0; ks <= last; ks += 2) {
    // buffer 0 holds ks, r1 holds ks+1, r0 is loading ks+2
    compute_stage<WF, XB, BM, BN>(sA0, sB0, wm, wn, g, c, acc);
    if (ks + 1 > last) break;
    store_stage<WF, XB, BM, BN>(sA1, sB1, (ks + 1) * kBK, r1);
    __syncthreads();
    load_stage<WF, XB, BM, BN>(p, m0, n0, min(ks + 3, last) * kBK, r1);
    // buffer 1 holds ks+1, r0 holds ks+2, r1 is loading ks+3
    compute_stage<WF, XB, BM, BN>(sA1, sB1, wm, wn, g, c, acc);
    if (ks + 2 > last) break;
    store_stage<WF, XB, BM, BN>(sA0, sB0, (ks + 2) * kBK, r0);
    __syncthreads();
    load_stage<WF, XB, BM, BN>(p, m0, n0, min(ks + 4, last) * kBK, r0);
  }
  }

  // Lane (g, c) holds out rows 4g .. 4g+3 of token c in each 16x16 tile.
  // A split K writes its fp32 partial sums to its own workspace slab.
  float* part = p.splits > 1 ? p.ws + (int64_t)split * p.M * p.N : nullptr;
#pragma unroll
  for (int i = 0; i < C::kTM; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * i + c;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
      const int n = n0 + wn * (BN / 2) + 16 * j + 4 * g;
      if (n >= p.N) continue;
      const float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2],
                                   acc[i][j][3]);
      if (part)
        *reinterpret_cast<float4*>(part + m * p.N + n) = v;
      else
        store4(p.out, m * p.N + n, v, OB);
    }
  }
}

// Sums the split-K partial slabs in a fixed order (deterministic).
template <bool OB>
__global__ __launch_bounds__(256) void proj_reduce_kernel(ProjParams p) {
  const int64_t total4 = p.M * p.N / 4;
  const int64_t slab4 = total4;
  const float4* ws = reinterpret_cast<const float4*>(p.ws);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < total4;
       i += (int64_t)gridDim.x * 256) {
    float4 a = ws[i];
    for (int s = 1; s < p.splits; ++s) {
      const float4 b = ws[s * slab4 + i];
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    store4(p.out, 4 * i, a, OB);
  }
}

// ---------------------------------------------------------- GEMV kernel --
// One wave per out row.  The row is walked in slices of 512 values; lane l
// takes values 8l .. 8l+7 of a slice (for Q4_K: 8 consecutive values of one
// sub-block, i.e. 8 quant bytes of one nibble half), decodes them to fp32
// and accumulates every token's dot product; a wave sum finishes each one.
template <int WF, bool XB, bool OB>
__global__ __launch_bounds__(256) void proj_gemv_kernel(ProjParams p) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= p.N) return;
  const int rows = (int)p.M;
  float acc[kGemvMaxRows];
#pragma unroll
  for (int m = 0; m < kGemvMaxRows; ++m) acc[m] = 0.f;
  const int slices = (p.K + 511) / 512;
#pragma unroll 4
  for (int it = 0; it < slices; ++it) {
    // Lanes past the row's end read its last 8 values and weigh them 0, so
    // that every load is unconditional and the unrolled loads overlap.
    const int kr = it * 512 + 8 * lane;
    const bool live = kr < p.K;
    const int k = live ? kr : p.K - 8;
    float w[8];
    if constexpr (WF == kFmtBf16) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
          static_cast<const uint16_t*>(p.w) + (int64_t)n * p.K + k);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(v[i] << 16);
        w[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
      }
    } else {
      const uint8_t* blk = static_cast<const uint8_t*>(p.w) +
                           (int64_t)n * (p.K / kQBlock) * kQBytes +
                           (int64_t)(k / kQBlock) * kQBytes;
      const int vb = k % kQBlock, j = vb / 32;
      const u32x4_t hdr = *reinterpret_cast<const u32x4_t*>(blk);
      const u32x2_t q = *reinterpret_cast<const u32x2_t*>(
          blk + 16 + 32 * (j >> 1) + (vb & 31));
      uint32_t sc, mn;
      scale_min(hdr[1], hdr[2], hdr[3], j, sc, mn);
      const float dsc = half_to_f32(hdr[0] & 0xffffu) * (float)sc;
      const float dmm = half_to_f32(hdr[0] >> 16) * (float)mn;
      const int shift = 4 * (j & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t byte = (q[i >> 2] >> (8 * (i & 3))) & 0xffu;
        w[i] = fmaf(dsc, (float)((byte >> shift) & 15u), -dmm);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = live ? w[i] : 0.f;
#pragma unroll
    for (int m = 0; m < kGemvMaxRows; ++m) {
      if (m >= rows) break;
      const int64_t off = (int64_t)m * p.K + k;
      const float4 x0 = load4(p.x, off, XB), x1 = load4(p.x, off + 4, XB);
      float a = acc[m];
      a = fmaf(w[0], x0.x, a);
      a = fmaf(w[1], x0.y, a);
      a = fmaf(w[2], x0.z, a);
      a = fmaf(w[3], x0.w, a);
      a = fmaf(w[4], x1.x, a);
      a = fmaf(w[5], x1.y, a);
      a = fmaf(w[6], x1.z, a);
      a = fmaf(w[7], x1.w, a);
      acc[m] = a;
    }
  }
#pragma unroll
  for (int m = 0; m < kGemvMaxRows; ++m) {
    if (m >= rows) break;
    const float t = group_sum<64>(acc[m]);
    if (lane == 0) store1(p.out, (int64_t)m * p.N + n, t, OB);
  }
}

template <int WF, bool XB, bool OB, int BM, int BN>
hipError_t launch_tiles(const ProjParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  proj_tile_kernel<WF, XB, OB, BM, BN>
      <<<(unsigned)(tiles * p.splits), 256, 0, s>>>(p);
  if (p.splits > 1) {
    int64_t blocks = (p.M * p.N / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    proj_reduce_kernel<OB><<<(unsigned)blocks, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

// Decodes the Q4_K weight into its two bf16 parts for the GEMM above 4096
// tokens: row n of p.wd holds the K high parts, then the K low parts, of W's
// row n -- the same fp32 values (one fma of exact terms) and the same split
// as the tile kernel's loader.  One thread per 8 consecutive values.
__global__ __launch_bounds__(256) void q4k_split_kernel(ProjParams p) {
  const int64_t per_row = p.K / 8;
  const int64_t units = (int64_t)p.N * per_row;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * 256) {
    const int64_t n = u / per_row;
    const int k = (int)(u - n * per_row) * 8;
    const uint8_t* blk = static_cast<const uint8_t*>(p.w) +
                         n * (int64_t)(p.K / kQBlock) * kQBytes +
                         (int64_t)(k / kQBlock) * kQBytes;
    const int within = k % kQBlock;
    const int step = within / kBK;          // 64-value step of the block
    const int l = within % kBK;             // < 32: low nibbles, else high
    const u32x4_t hdr = *reinterpret_cast<const u32x4_t*>(blk);
    const u32x2_t q = *reinterpret_cast<const u32x2_t*>(blk + 16 + 32 * step + (l & 31));
    const SubScales sc = sub_scales(hdr, step);
    float v0[8], v1[8];
    decode_word(q[0], sc, v0, v1);
    decode_word(q[1], sc, v0 + 4, v1 + 4);
    u32x4_t parts[2];
    split8<2>(l < 32 ? v0 : v1, parts);
    uint16_t* row = p.wd + n * 2 * (int64_t)p.K;
    *reinterpret_cast<u32x4_t*>(row + k) = parts[0];
    *reinterpret_cast<u32x4_t*>(row + p.K + k) = parts[1];
  }
}

template <int WF, bool XB, bool OB>
hipError_t launch_typed(const ProjParams& p, ProjKernel k, hipStream_t s) {
  switch (k) {
    case ProjKernel::kGemv:
      proj_gemv_kernel<WF, XB, OB><<<(p.N + 3) / 4, 256, 0, s>>>(p);
      return hipGetLastError();
    case ProjKernel::kTile32x64:
      return launch_tiles<WF, XB, OB, 32, 64>(p, s);
    case ProjKernel::kTile64x64:
      return launch_tiles<WF, XB, OB, 64, 64>(p, s);
    case ProjKernel::kTile128x128:
      // Two 128 x 128 buffers of three-part x and weight exceed the LDS;
      // the planner sends that case to 64 x 64 tiles.
      if constexpr (WF == kFmtQ4K && !XB) return hipErrorInvalidValue;
      else return launch_tiles<WF, XB, OB, 128, 128>(p, s);
    case ProjKernel::kGemm:
      if constexpr (WF == kFmtBf16 && XB) {
        return launch_gemm_bf16(p, s);
      } else if constexpr (WF == kFmtQ4K && XB) {
        if (!p.wd) return hipErrorInvalidValue;
        const int64_t units = (int64_t)p.N * (p.K / 8);
        const int64_t blocks = min((units + 255) / 256, (int64_t)4096);
        q4k_split_kernel<<<(unsigned)blocks, 256, 0, s>>>(p);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_gemm_bf16(p, s);
      } else {
        return hipErrorInvalidValue;
      }
  }
  return hipErrorInvalidValue;
}

template <int WF>
hipError_t launch_w(const ProjParams& p, ProjKernel k, hipStream_t s) {
  if (p.x_bf16)
    return p.out_bf16 ? launch_typed<WF, true, true>(p, k, s)
                      : launch_typed<WF, true, false>(p, k, s);
  return p.out_bf16 ? launch_typed<WF, false, true>(p, k, s)
                    : launch_typed<WF, false, false>(p, k, s);
}


// ------------------------------------------------ FP8 / MXFP4 (W8A8, W4A4) --
// Activation quantization.  FP8: one power-of-two scale per token, the
// smallest 2^e with max|x| / 2^e <= 448 (e from the exponent of max|x|:
// max|x| = f 2^E with f in [0.5, 1) gives e = E - 9 when f <= 0.875, else
// E - 8; at least -126), then E4M3 codes of x / 2^e, rounded to nearest
// even.  MXFP4: per block of 32
// values along K, the E8M0 scale 127 + floor(log2 max|v|) - 2 (clamped to
// 0..254; 127 for an all-zero block), then E2M1 codes of v / scale, nearest
// even, saturating at 6.  Divisions are by powers of two, hence exact.

// Four values to E4M3 codes (byte i holds value i) and eight to E2M1 codes
// (nibble i holds value i), by the conversion instructions, which round to
// nearest even; the inputs are already divided by their power-of-two scale
// and lie within the formats' ranges (|x| <= 448 for E4M3; E2M1 saturates
// at 6).  A zero's E4M3 code keeps its sign; an exact zero's E2M1 code is
// the positive one (x + 0 turns -0 into +0), while a negative value that
// rounds to zero keeps its sign.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  const int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
__device__ __forceinline__ uint32_t e2m1x8(const float (&x)[8]) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] + 0.0f, x[1] + 0.0f, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] + 0.0f, x[3] + 0.0f, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] + 0.0f, x[5] + 0.0f, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] + 0.0f, x[7] + 0.0f, 1.0f, 3);
  return w;
}

template <bool XB>
__device__ __forceinline__ void load8(const void* x, int64_t off, float* v) {
  const float4 a = load4(x, off, XB), b = load4(x, off + 4, XB);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One wave per token row: a pass for max|x|, then a pass that encodes (the
// row is back in cache by then).  Lanes past the row's end read its last 8
// values and store nothing.
template <bool XB>
__global__ __launch_bounds__(256) void quant_fp8_kernel(QuantParams q) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= q.M) return;
  const int64_t base = row * q.K;
  float amax = 0.f;
  for (int k0 = 0; k0 < q.K; k0 += 512) {
    const int k = k0 + 8 * lane;
    const bool live = k < q.K;
    float v[8];
    load8<XB>(q.x, base + (live ? k : q.K - 8), v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, live ? fabsf(v[i]) : 0.f);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  int e = 0;
  if (amax > 0.f) {
    int E;
    const float f = frexpf(amax, &E);
    e = f <= 0.875f ? E - 9 : E - 8;
    e = max(e, -126);
  }
  if (lane == 0) static_cast<float*>(q.scales)[row] = ldexpf(1.0f, e);
  for (int k0 = 0; k0 < q.K; k0 += 512) {
    const int k = k0 + 8 * lane;
    if (k >= q.K) break;
    float v[8];
    load8<XB>(q.x, base + k, v);
    const uint32_t w0 = e4m3x4(ldexpf(v[0], -e), ldexpf(v[1], -e),
                               ldexpf(v[2], -e), ldexpf(v[3], -e));
    const uint32_t w1 = e4m3x4(ldexpf(v[4], -e), ldexpf(v[5], -e),
                               ldexpf(v[6], -e), ldexpf(v[7], -e));
    *reinterpret_cast<u32x2_t*>(q.codes + base + k) = u32x2_t{w0, w1};
  }
}

// One wave per token row with the row held in registers (up to
// kQuantChunks chunks of 8 values per lane, K <= 4096): one read of x, a
// wave reduction for max|x|, then the encode.
constexpr int kQuantChunks = 8;

template <bool XB>
__global__ __launch_bounds__(256) void quant_fp8_row_kernel(QuantParams q) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= q.M) return;
  const int64_t base = row * q.K;
  const int chunks = q.K / 8;
  float v[kQuantChunks][8];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < kQuantChunks; ++j) {
    const int ch = lane + 64 * j;
    const bool live = ch < chunks;
    load8<XB>(q.x, base + 8 * (live ? ch : chunks - 1), v[j]);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, live ? fabsf(v[j][i]) : 0.f);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  int e = 0;
  if (amax > 0.f) {
    int E;
    const float f = frexpf(amax, &E);
    e = f <= 0.875f ? E - 9 : E - 8;
    e = max(e, -126);
  }
  if (lane == 0) static_cast<float*>(q.scales)[row] = ldexpf(1.0f, e);
#pragma unroll
  for (int j = 0; j < kQuantChunks; ++j) {
    const int ch = lane + 64 * j;
    if (ch < chunks) {
      const uint32_t w0 = e4m3x4(ldexpf(v[j][0], -e), ldexpf(v[j][1], -e),
                                 ldexpf(v[j][2], -e), ldexpf(v[j][3], -e));
      const uint32_t w1 = e4m3x4(ldexpf(v[j][4], -e), ldexpf(v[j][5], -e),
                                 ldexpf(v[j][6], -e), ldexpf(v[j][7], -e));
      *reinterpret_cast<u32x2_t*>(q.codes + base + 8 * ch) = u32x2_t{w0, w1};
    }
  }
}

// One thread per 8 values; the 4 threads of a 32-value block are adjacent
// lanes and share its max through two lane swaps (most threads in flight:
// small inputs).
template <bool XB>
__global__ __launch_bounds__(256) void quant_mxfp4_quad_kernel(QuantParams q) {
  const int64_t units = q.M * q.K / 8;
  for (int64_t u = blockIdx.x * 256ll + threadIdx.x; u < units;
       u += (int64_t)gridDim.x * 256) {
    const int64_t row = u / (q.K / 8);
    const int k = (int)(u - row * (q.K / 8)) * 8;
    float v[8];
    load8<XB>(q.x, row * q.K + k, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    int s = 127;
    if (amax > 0.f) {
      int E;
      frexpf(amax, &E);
      s = min(254, max(0, 124 + E));
    }
    float sv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[i], 127 - s);
    const uint32_t w = e2m1x8(sv);
    *reinterpret_cast<uint32_t*>(q.codes + row * (q.K / 2) + k / 2) = w;
    if ((k & 31) == 0)
      static_cast<uint8_t*>(q.scales)[row * (q.K / 32) + k / 32] = (uint8_t)s;
  }
}

// One thread per 32-value block: its maximum, scale and 16 bytes of codes
// (more work per thread: large inputs).
template <bool XB>
__global__ __launch_bounds__(256) void quant_mxfp4_kernel(QuantParams q) {
  const int64_t blocks = q.M * q.K / 32;
  for (int64_t bi = blockIdx.x * 256ll + threadIdx.x; bi < blocks;
       bi += (int64_t)gridDim.x * 256) {
    const int64_t row = bi / (q.K / 32);
    const int k = (int)(bi - row * (q.K / 32)) * 32;
    float v[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) load8<XB>(q.x, row * q.K + k + 8 * j, v + 8 * j);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    int s = 127;
    if (amax > 0.f) {
      int E;
      frexpf(amax, &E);
      s = min(254, max(0, 124 + E));
    }
    u32x4_t w;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[8 * j + i], 127 - s);
      w[j] = e2m1x8(sv);
    }
    *reinterpret_cast<u32x4_t*>(q.codes + row * (q.K / 2) + k / 2) = w;
    static_cast<uint8_t*>(q.scales)[bi] = (uint8_t)s;
  }
}

// Matrix-core tile kernel over byte operands (v_mfma_scale_f32_16x16x128_
// f8f6f4).  Operand layout (checked on the hardware): lane (g, c) supplies
// row c, values 32g .. 32g+31 of the 128-value K slice -- 32 bytes of E4M3
// or 16 bytes of E2M1 (even value in the low nibble) -- and, for E2M1, the
// E8M0 scale of that row's 32-value block g; lane (g, c) receives D[4g+i][c].
// A K-step is one 128-byte row slice per operand row: 128 FP8 values (one
// instruction) or 256 FP4 values (two).  FP8 runs the instruction with unit
// scales and applies the per-token and per-row scales to the fp32 result.
template <int FMT, int BM, int BN>
struct LpCfg {
  static constexpr bool kFp4 = FMT == kFmtMxfp4;
  static constexpr int kKS = kFp4 ? 256 : 128;      // values per step
  static constexpr int kTM = BM / 32, kTN = BN / 32;
  static constexpr int kAG = BM * 8 / 256, kBG = BN * 8 / 256;
  static constexpr int kA = BM * 64, kB = BN * 64;  // uint16 per tile
  static constexpr int kAS = kFp4 ? BM * 8 : 0;     // scale bytes per tile
  static constexpr int kBS = kFp4 ? BN * 8 : 0;
  static constexpr int kStage = 2 * (kA + kB) + kAS + kBS;   // bytes
  static constexpr bool kDB = 2 * kStage <= 80 * 1024;
};

template <int FMT, int BM, int BN>
struct LpStage {
  using C = LpCfg<FMT, BM, BN>;
  u32x4_t xa[C::kAG];
  u32x4_t wb[C::kBG];
  u32x2_t sc;                       // MXFP4: 8 scale bytes of one row
};

template <int FMT, int BM, int BN>
__device__ __forceinline__ void lp_load(const ProjParams& p, int64_t m0,
                                        int n0, int ks,
                                        LpStage<FMT, BM, BN>& st) {
  using C = LpCfg<FMT, BM, BN>;
  const int tid = threadIdx.x;
  const int64_t rowb = C::kFp4 ? p.K / 2 : p.K;    // code bytes per row
  const int64_t kb = (int64_t)ks * 128;             // byte offset of step
#pragma unroll
  for (int i = 0; i < C::kAG; ++i) {
    const int G = tid + 256 * i;
    const int64_t row = min(m0 + (G >> 3), p.M - 1);
    st.xa[i] = *reinterpret_cast<const u32x4_t*>(p.xq + row * rowb + kb +
                                                 16 * (G & 7));
  }
#pragma unroll
  for (int i = 0; i < C::kBG; ++i) {
    const int G = tid + 256 * i;
    const int64_t row = min((int64_t)n0 + (G >> 3), (int64_t)p.N - 1);
    st.wb[i] = *reinterpret_cast<const u32x4_t*>(
        static_cast<const uint8_t*>(p.w) + row * rowb + kb + 16 * (G & 7));
  }
  if constexpr (C::kFp4) {
    // Threads 0 .. BM-1 fetch token rows' 8 block scales, BM .. BM+BN-1
    // the weight rows'; the rest re-read a valid row (unused).
    const int r = min(tid, BM + BN - 1);
    const int64_t nb = p.K / 32;
    const uint8_t* src;
    if (r < BM)
      src = static_cast<const uint8_t*>(p.xs) + min(m0 + r, p.M - 1) * nb;
    else
      src = static_cast<const uint8_t*>(p.wscale) +
            min((int64_t)n0 + (r - BM), (int64_t)p.N - 1) * nb;
    st.sc = *reinterpret_cast<const u32x2_t*>(src + 8 * ks);
  }
}

template <int FMT, int BM, int BN>
__device__ __forceinline__ void lp_store(uint8_t* buf,
                                         const LpStage<FMT, BM, BN>& st) {
  using C = LpCfg<FMT, BM, BN>;
  uint16_t* sA = reinterpret_cast<uint16_t*>(buf);
  uint16_t* sB = sA + C::kA;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::kAG; ++i) {
    const int G = tid + 256 * i;
    *reinterpret_cast<u32x4_t*>(sA + sw(G >> 3, 8 * (G & 7))) = st.xa[i];
  }
#pragma unroll
  for (int i = 0; i < C::kBG; ++i) {
    const int G = tid + 256 * i;
    *reinterpret_cast<u32x4_t*>(sB + sw(G >> 3, 8 * (G & 7))) = st.wb[i];
  }
  if constexpr (C::kFp4) {
    if (tid < BM + BN)
      *reinterpret_cast<u32x2_t*>(buf + 2 * (C::kA + C::kB) + 8 * tid) = st.sc;
  }
}

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

template <int FMT, int BM, int BN>
__device__ __forceinline__ void lp_compute(
    const uint8_t* buf, int wm, int wn, int g, int c,
    f32x4_t (&acc)[LpCfg<FMT, BM, BN>::kTM][LpCfg<FMT, BM, BN>::kTN]) {
  using C = LpCfg<FMT, BM, BN>;
  const uint16_t* sA = reinterpret_cast<const uint16_t*>(buf);
  const uint16_t* sB = sA + C::kA;
  const uint8_t* sS = buf + 2 * (C::kA + C::kB);   // [BM + BN][8] scales
  constexpr int kInstr = C::kFp4 ? 2 : 1;
#pragma unroll
  for (int kc = 0; kc < kInstr; ++kc) {
    i32x8_t xf[C::kTM], wf[C::kTN];
    int xsc[C::kTM], wsc[C::kTN];
#pragma unroll
    for (int i = 0; i < C::kTM; ++i) {
      const int r = wm * (BM / 2) + 16 * i + c;
      if constexpr (C::kFp4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sA + sw(r, 8 * (4 * kc + g)));
        xf[i] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        xsc[i] = sS[8 * r + 4 * kc + g];
      } else {
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(sA + sw(r, 8 * (2 * g)));
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(sA + sw(r, 8 * (2 * g + 1)));
        xf[i] = i32x8_t{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                        (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
        xsc[i] = 127;
      }
    }
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
      const int r = wn * (BN / 2) + 16 * j + c;
      if constexpr (C::kFp4) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(sB + sw(r, 8 * (4 * kc + g)));
        wf[j] = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
        wsc[j] = sS[8 * (BM + r) + 4 * kc + g];
      } else {
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(sB + sw(r, 8 * (2 * g)));
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(sB + sw(r, 8 * (2 * g + 1)));
        wf[j] = i32x8_t{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                        (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
        wsc[j] = 127;
      }
    }
    constexpr int kF = C::kFp4 ? 4 : 0;       // instruction format field
#pragma unroll
    for (int i = 0; i < C::kTM; ++i)
#pragma unroll
      for (int j = 0; j < C::kTN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf[j], xf[i], acc[i][j], kF, kF, 0, wsc[j], 0, xsc[i]);
  }
}

template <int FMT, bool OB, int BM, int BN>
__global__ __launch_bounds__(256) void lp_tile_kernel(ProjParams p) {
  using C = LpCfg<FMT, BM, BN>;
  __shared__ __align__(16) uint8_t smem[(C::kDB ? 2 : 1) * C::kStage];
  uint8_t* const buf0 = smem;
  uint8_t* const buf1 = smem + (C::kDB ? C::kStage : 0);

  const int tiles_m = (int)((p.M + BM - 1) / BM);
  const int tiles_n = (p.N + BN - 1) / BN;
  const int tiles = tiles_m * tiles_n;
  const int nb = gridDim.x;
  const int b = blockIdx.x;
  const int lid = (nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  const int split = lid / tiles, t = lid % tiles;
  constexpr int kGroup = 8;
  const int grp = t / (kGroup * tiles_n), in = t % (kGroup * tiles_n);
  const int gm = min(kGroup, tiles_m - grp * kGroup);
  const int64_t m0 = (int64_t)(grp * kGroup + in % gm) * BM;
  const int n0 = (in / gm) * BN;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;
  f32x4_t acc[C::kTM][C::kTN];
#pragma unroll
  for (int i = 0; i < C::kTM; ++i)
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int steps = p.K / C::kKS / p.splits;
  const int ks0 = split * steps, last = ks0 + steps - 1;
  if constexpr (!C::kDB) {
    LpStage<FMT, BM, BN> st;
    lp_load<FMT, BM, BN>(p, m0, n0, ks0, st);
    for (int ks = ks0; ks <= last; ++ks) {
      if (ks > ks0) __syncthreads();
      lp_store<FMT, BM, BN>(buf0, st);
      __syncthreads();
      lp_load<FMT, BM, BN>(p, m0, n0, min(ks + 1, last), st);
      lp_compute<FMT, BM, BN>(buf0, wm, wn, g, c, acc);
    }
  } else {
    LpStage<FMT, BM, BN> r0, r1;
    lp_load<FMT, BM, BN>(p, m0, n0, ks0, r0);
    lp_load<FMT, BM, BN>(p, m0, n0, min(ks0 + 1, last), r1);
    lp_store<FMT, BM, BN>(buf0, r0);
    __syncthreads();
    lp_load<FMT, BM, BN>(p, m0, n0, min(ks0 + 2, last), r0);
    for (int ks = ks0; ks <= last; ks += 2) {
      lp_compute<FMT, BM, BN>(buf0, wm, wn, g, c, acc);
      if (ks + 1 > last) break;
      lp_store<FMT, BM, BN>(buf1, r1);
      __syncthreads();
      lp_load<FMT, BM, BN>(p, m0, n0, min(ks + 3, last), r1);
      lp_compute<FMT, BM, BN>(buf1, wm, wn, g, c, acc);
      if (ks + 2 > last) break;
      lp_store<FMT, BM, BN>(buf0, r0);
      __syncthreads();
      lp_load<FMT, BM, BN>(p, m0, n0, min(ks + 4, last), r0);
    }
  }

  float* part = p.splits > 1 ? p.ws + (int64_t)split * p.M * p.N : nullptr;
#pragma unroll
  for (int i = 0; i < C::kTM; ++i) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * i + c;
    if (m >= p.M) continue;
    const float xsc = C::kFp4 ? 1.0f : static_cast<const float*>(p.xs)[m];
#pragma unroll
    for (int j = 0; j < C::kTN; ++j) {
      const int n = n0 + wn * (BN / 2) + 16 * j + 4 * g;
      if (n >= p.N) continue;
      float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2],
                             acc[i][j][3]);
      if constexpr (!C::kFp4) {
        const float4 ws4 =
            *reinterpret_cast<const float4*>(static_cast<const float*>(p.wscale) + n);
        v.x *= xsc * ws4.x;
        v.y *= xsc * ws4.y;
        v.z *= xsc * ws4.z;
        v.w *= xsc * ws4.w;
      }
      if (part)
        *reinterpret_cast<float4*>(part + m * p.N + n) = v;
      else
        store4(p.out, m * p.N + n, v, OB);
    }
  }
}

template <int FMT, bool OB, int BM, int BN>
hipError_t launch_lp_tiles(const ProjParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  lp_tile_kernel<FMT, OB, BM, BN><<<(unsigned)(tiles * p.splits), 256, 0, s>>>(p);
  if (p.splits > 1) {
    int64_t blocks = (p.M * p.N / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    proj_reduce_kernel<OB><<<(unsigned)blocks, 256, 0, s>>>(p);
  }
  return hipGetLastError();
}

template <int FMT, bool OB>
hipError_t launch_lp(const ProjParams& p, ProjKernel k, hipStream_t s) {
  switch (k) {
    case ProjKernel::kTile32x64: return launch_lp_tiles<FMT, OB, 32, 64>(p, s);
    case ProjKernel::kTile64x64: return launch_lp_tiles<FMT, OB, 64, 64>(p, s);
    case ProjKernel::kTile128x128: return launch_lp_tiles<FMT, OB, 128, 128>(p, s);
    case ProjKernel::kGemm: return launch_gemm_lp(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

namespace {
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

ProjPlan plan_out_proj(int64_t M, int32_t K, int32_t N, int32_t wfmt,
                       bool x_f32) {
  ProjPlan pl{ProjKernel::kGemv, 1, 0, 0, 0, 0, 0};
  const bool lp = wfmt == kFmtFp8 || wfmt == kFmtMxfp4;
  if (lp) {
    // Quantized activations come first in the workspace.
    const size_t codes = wfmt == kFmtFp8 ? (size_t)M * K : (size_t)M * K / 2;
    const size_t scales =
        wfmt == kFmtFp8 ? (size_t)M * sizeof(float) : (size_t)M * K / 32;
    pl.xq_off = 0;
    pl.xs_off = align256(codes);
    pl.slab_off = pl.xs_off + align256(scales);
    pl.ws_bytes = pl.slab_off;
  }
  if (!lp && M <= kGemvMaxRows) return pl;
  if (M > 4096) {
    if ((lp || (wfmt == kFmtBf16 && !x_f32)) && K <= kGemmMaxK) {
      pl.kernel = ProjKernel::kGemm;
    } else if (wfmt == kFmtQ4K && !x_f32 && 2 * (int64_t)K <= kGemmMaxK) {
      // The weight decoded once into its two bf16 parts, then the GEMM.
      pl.kernel = ProjKernel::kGemm;
      pl.wd_off = 0;
      pl.ws_bytes = align256((size_t)N * K * 4);
    } else {
      pl.kernel = (wfmt == kFmtQ4K && x_f32) ? ProjKernel::kTile64x64
                                             : ProjKernel::kTile128x128;
    }
    return pl;
  }
  // Up to a few thousand tokens the tile grid alone is too small to fill
  // the chip; split K (in powers of two, at least 4 steps per range) until
  // about 512 workgroups run.
  const int BM = M <= 64 ? 32 : 64;
  pl.kernel = M <= 64 ? ProjKernel::kTile32x64 : ProjKernel::kTile64x64;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + 63) / 64);
  const int step = wfmt == kFmtFp8 ? 128 : (wfmt == kFmtMxfp4 ? 256 : kBK);
  const int nK = K / step;
  while (pl.splits < 16 && tiles * pl.splits * 2 <= 512 &&
         nK % (2 * pl.splits) == 0 && nK / (2 * pl.splits) >= 4)
    pl.splits *= 2;
  if (pl.splits > 1)
    pl.ws_bytes = pl.slab_off + (size_t)pl.splits * M * N * sizeof(float);
  return pl;
}

// Up to this many MXFP4 blocks the quad kernel (4 threads per block) keeps
// more threads in flight; beyond, one thread per block does more per thread.
constexpr int64_t kMxQuadBlocks = 1 << 18;

hipError_t launch_quantize(const QuantParams& q, hipStream_t stream) {
  if (q.M == 0) return hipSuccess;
  if (q.fmt == kFmtFp8) {
    const unsigned blocks = (unsigned)((q.M + 3) / 4);
    if (q.K <= 8 * 64 * kQuantChunks) {
      if (q.x_bf16) quant_fp8_row_kernel<true><<<blocks, 256, 0, stream>>>(q);
      else quant_fp8_row_kernel<false><<<blocks, 256, 0, stream>>>(q);
    } else {
      if (q.x_bf16) quant_fp8_kernel<true><<<blocks, 256, 0, stream>>>(q);
      else quant_fp8_kernel<false><<<blocks, 256, 0, stream>>>(q);
    }
  } else if (q.M * q.K / 32 < kMxQuadBlocks) {
    const int64_t blocks = (q.M * q.K / 8 + 255) / 256;
    if (q.x_bf16) quant_mxfp4_quad_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(q);
    else quant_mxfp4_quad_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(q);
  } else {
    int64_t blocks = (q.M * q.K / 32 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (q.x_bf16) quant_mxfp4_kernel<true><<<(unsigned)blocks, 256, 0, stream>>>(q);
    else quant_mxfp4_kernel<false><<<(unsigned)blocks, 256, 0, stream>>>(q);
  }
  return hipGetLastError();
}

hipError_t launch_out_proj(const ProjParams& p, hipStream_t stream) {
  if (p.M == 0) return hipSuccess;
  // One workgroup per tile and range: the count must fit a 1-D grid.
  if (((p.M + 31) / 32) * ((p.N + 63) / 64) * p.splits > (int64_t)INT32_MAX)
    return hipErrorInvalidValue;
  const ProjKernel k = plan_out_proj(p.M, p.K, p.N, p.wfmt, p.x_bf16 == 0).kernel;
  if (p.wfmt == kFmtFp8 || p.wfmt == kFmtMxfp4) {
    QuantParams q{p.x, p.xq, p.xs, p.M, p.K, p.x_bf16, p.wfmt};
    const hipError_t e = launch_quantize(q, stream);
    if (e != hipSuccess) return e;
    if (p.wfmt == kFmtFp8)
      return p.out_bf16 ? launch_lp<kFmtFp8, true>(p, k, stream)
                        : launch_lp<kFmtFp8, false>(p, k, stream);
    return p.out_bf16 ? launch_lp<kFmtMxfp4, true>(p, k, stream)
                      : launch_lp<kFmtMxfp4, false>(p, k, stream);
  }
  return p.wfmt == kFmtQ4K ? launch_w<kFmtQ4K>(p, k, stream)
                           : launch_w<kFmtBf16>(p, k, stream);
}

}  // namespace gdn
