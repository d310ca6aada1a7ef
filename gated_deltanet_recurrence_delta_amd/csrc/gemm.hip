// gemm.hip -- the output projection for long prefills as 256 x 256 tile
// GEMMs: y[m, :] = W x[m, :] with W [N out rows, K] and x [M, K] in dense
// bf16, or in FP8 / MXFP4 codes (further down), fp32 accumulation ("Red
// Lite dev15d -- DeltaNet gated tail + Q4_K output projection", Pinned graph
// semantics step 6, with the weight kept dense or in low-precision codes).
//
// A workgroup of 8 waves (two per SIMD) computes 256 tokens x 256 out rows;
// wave (wm, wn) holds tokens 128 wm .. +127 and rows 64 wn .. +63, 8 x 4
// tiles of 16 x 16 on v_mfma_f32_16x16x32_bf16, K advancing 64 per step.
// Operands go straight from global memory into LDS with direct-to-LDS loads
// (global_load_lds_dwordx4: lane l's 16 bytes land at the wave-uniform LDS
// base + 16 l), one step ahead into two 64 KiB buffers, with no register
// staging.  A load covers 8 tile rows of 128 bytes (whole lines); each lane
// fetches the global granule that the tile swizzle places at its LDS slot.
// Each step is two halves of 32 K values: the fragment reads of one half are
// interleaved with the matrix-core work of the half before, and the single
// barrier per step sits between the halves.
//
// Built with the matrix-core instructions in their VGPR form (a per-file
// compiler option): the 128 accumulators per lane then stay in place instead
// of being copied between accumulation and vector registers.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_proj.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;             // K values per step

__device__ __forceinline__ f32x4_t mfma32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kGM = 256;            // tokens per workgroup
constexpr int kGN = 256;            // out rows per workgroup
constexpr int kGWaves = 8;          // two per SIMD, 128 tokens x 64 rows each
constexpr int kWavesN = kGWaves / 2;          // waves across the out rows
constexpr int kWR = kGN / kWavesN;            // out rows per wave
constexpr int kTJ = kWR / 16;                 // 16-row tiles per wave
constexpr int kGStages = 2;         // LDS buffers (loads one step ahead)
constexpr int kGLoads = (kGM + kGN) / 8 / kGWaves;   // direct loads per wave and step

// Tile rows hold 64 bf16 (eight 16-byte granules); granule q of row r sits
// at slot q ^ ((r >> 1) & 7), so the 16 lanes of a fragment read (16
// consecutive rows, one granule each) cover the 64 banks once.
__device__ __forceinline__ int gsw(int r, int q) {
  return r * kBK + ((q ^ ((r >> 1) & 7)) << 3);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ lds_ptr_t lds_addr(const void* p) {
  return (lds_ptr_t)(uintptr_t)(uint32_t)(uintptr_t)p;
}

// Direct-to-LDS loads of 16 and 4 bytes a lane: lane l's bytes land at
// lds + 16 l (lds + 4 l).  Plain functions: inside the kernel template the
// builtin's size operand keeps the host pass from emitting the launch stub.
__device__ __forceinline__ void dma16(const char* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds_addr(lds), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const char* src, void* lds) {
  __builtin_amdgcn_global_load_lds(src, lds_addr(lds), 4, 0, 0);
}

// s_waitcnt immediate: at most n vector memory operations outstanding and
// no LDS operation (vmcnt bits [3:0] and [15:14], lgkmcnt 0, expcnt not
// waited for).
constexpr int gwait(int n) { return ((n >> 4) << 14) | 0x0070 | (n & 15); }
// s_waitcnt immediate: no LDS operation outstanding (vmcnt and expcnt at
// their maxima, i.e. not waited for).
constexpr int kLdsDone = (3 << 14) | 0x0070 | 15;

// First token and out row of this workgroup's tile.  Tile order as in the
// projection's tile kernels: each XCD takes a contiguous run of tile ids,
// grouped 8 token panels at a time.
__device__ __forceinline__ void tile_origin(const ProjParams& p, int64_t& m0,
                                            int& n0) {
  const int tiles_m = (int)((p.M + kGM - 1) / kGM);
  const int tiles_n = (p.N + kGN - 1) / kGN;
  const int nb = gridDim.x, b = blockIdx.x;
  const int t = (nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  constexpr int kGroup = 8;
  const int grp = t / (kGroup * tiles_n), in = t % (kGroup * tiles_n);
  const int gm = min(kGroup, tiles_m - grp * kGroup);
  m0 = (int64_t)(grp * kGroup + in % gm) * kGM;
  n0 = (in / gm) * kGN;
}

template <bool OB>
__global__ __launch_bounds__(64 * kGWaves) void gemm_bf16_kernel(ProjParams p) {
  __shared__ __align__(16) uint16_t smem[kGStages][(kGM + kGN) * kBK];

  int64_t m0;
  int n0;
  tile_origin(p, m0, n0);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // Sources of this lane's loads: load i of wave w covers rows
  // 8 (8 i + w) .. +7 of the combined tile (x rows 0..255, then W rows),
  // as a byte offset from the tile's first x or W row (a wave-uniform base,
  // so the load forms the address itself); rows past M or N repeat the last
  // one (valid addresses, never stored).
  // A decoded Q4_K weight (p.wd) has rows of 2 K parts, high then low; the
  // x rows are then walked twice, so each part meets the same activations.
  const int wk = p.wd ? 2 * p.K : p.K;
  const char* xb = static_cast<const char*>(p.x) + m0 * p.K * 2;
  const char* wb = static_cast<const char*>(p.wd ? static_cast<const void*>(p.wd) : p.w) +
                   (int64_t)n0 * wk * 2;
  uint32_t off[kGLoads];
#pragma unroll
  for (int i = 0; i < kGLoads; ++i) {
    const int cr = 8 * (kGWaves * i + wave) + (lane >> 3);
    const int q = (lane & 7) ^ ((cr >> 1) & 7);
    const int r = cr < kGM ? (int)min((int64_t)cr, p.M - 1 - m0)
                           : min(cr - kGM, p.N - 1 - n0);
    off[i] = (uint32_t)r * (uint32_t)(cr < kGM ? p.K : wk) * 2u + 16u * q;
  }
  const int xsteps = p.K / kBK, steps = wk / kBK;
  auto issue = [&](int s, int buf) {
    const int st = min(s, steps - 1);
    const int kx = (st >= xsteps ? st - xsteps : st) * kBK * 2, kw = st * kBK * 2;
#pragma unroll
    for (int i = 0; i < kGLoads; ++i)
      dma16((8 * kGWaves * i < kGM ? xb + kx : wb + kw) + off[i],
            &smem[buf][8 * (kGWaves * i + wave) * kBK]);
  };
  // Wait for this wave's loads of the next step (those of the step after
  // stay in flight) and its LDS reads, then for every wave's. A release
  // fence would wait for the loads still in flight as well; the empty asm
  // statements keep the compiler from moving memory accesses across.
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(gwait(kGLoads * (kGStages - 2)));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  f32x4_t acc[8][kTJ];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Fragments of one 32-wide K slice: lane (g, c) holds K values
  // 8 g .. 8 g + 7 of token row 16 i + c and of out row 16 j + c.
  struct Frags {
    bf16x8_t x[8], w[kTJ];
  };
  auto read = [&](Frags& f, int buf, int kc) {
    const uint16_t* sA = smem[buf];
    const uint16_t* sB = smem[buf] + kGM * kBK;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      f.x[i] = *reinterpret_cast<const bf16x8_t*>(sA + gsw(wm * 128 + 16 * i + c, 4 * kc + g));
#pragma unroll
    for (int j = 0; j < kTJ; ++j)
      f.w[j] = *reinterpret_cast<const bf16x8_t*>(sB + gsw(wn * kWR + 16 * j + c, 4 * kc + g));
  };
  auto mma = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < kTJ; ++j)
        // D[n][m]: W rows on the A side, tokens on the B side.
        acc[i][j] = mfma32(f.w[j], f.x[i], acc[i][j]);
  };
  // Scheduling of the preceding reads and matrix-core work: one fragment
  // read (group mask 0x100, LDS reads) after every two matrix-core
  // instructions (mask 0x008), the rest of the matrix-core work after.
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < 8 + kTJ; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8 * kTJ - 2 * (8 + kTJ), 0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Every step issues exactly kGLoads loads (past the last step they re-read
  // it into a buffer nobody reads again), so the wait count is exact.  The
  // fragment reads of each half step are in flight during the matrix-core
  // work of the half before it; the barrier sits between the two halves,
  // after the last read of the step's buffer, which the loads issued right
  // after it then refill.
#pragma unroll
  for (int st = 0; st + 1 < kGStages; ++st) issue(st, st);
  sync();
  issue(kGStages - 1, kGStages - 1);
  Frags f0, f1;
  read(f0, 0, 0);
  int cur = 0;
  for (int s = 0; s < steps; ++s) {
    // The reads of f0 were issued before the previous half step's
    // matrix-core work and are done; saying so here keeps the compiler from
    // waiting for the reads of f1 as well before using f0.
    __builtin_amdgcn_s_waitcnt(kLdsDone);
    __builtin_amdgcn_sched_barrier(0);
    read(f1, cur, 1);
    mma(f0);
    interleave();
    sync();
    issue(s + kGStages, cur);
    cur = cur == kGStages - 1 ? 0 : cur + 1;
    __builtin_amdgcn_sched_barrier(0);
    read(f0, cur, 0);
    mma(f1);
    interleave();
  }
  // Drain the loads issued past the last step before the workgroup ends.
  __builtin_amdgcn_s_waitcnt(gwait(0));

  // Lane (g, c) holds out rows 4g .. 4g+3 of token c in each 16x16 tile.
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + wm * 128 + 16 * i + c;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < kTJ; ++j) {
      const int n = n0 + wn * kWR + 16 * j + 4 * g;
      if (n >= p.N) continue;
      store4(p.out, m * p.N + n, make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2],
                                             acc[i][j][3]), OB);
    }
  }
}


// ------------------------------------------------- FP8 / MXFP4 codes GEMM --
// The same tile, waves and direct-to-LDS loads over byte codes: a 128-byte
// row slice per step holds 128 E4M3 values (one v_mfma_scale_f32_16x16x128_
// f8f6f4) or 256 E2M1 values (two).  Operand layout of that instruction:
// lane (g, c) supplies row c, values 32 g .. 32 g + 31 of the 128-value
// slice -- 32 bytes of E4M3 (granules 2 g and 2 g + 1 of the row slice) or 16
// bytes of E2M1 (granule 4 kc + g of instruction kc, even value in the low
// nibble) -- and, for E2M1, the E8M0 scale of that row's 32-value block.
// MXFP4 block scales reach LDS through two more direct loads per wave and
// step (4 bytes a lane: half of a row's 8 scales for the step).  Both
// formats pipeline their fragment reads across token halves of each
// instruction (below).  FP8 runs the instruction with unit scales and applies the per-token and
// per-row scales to the fp32 result.
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// D += A B with E8M0 block scales sa, sb; F: operand format (0 E4M3, 4 E2M1).
template <int F>
__device__ __forceinline__ f32x4_t mfma_scaled(i32x8_t a, i32x8_t b, f32x4_t c,
                                               int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, F, F, 0, sa, 0, sb);
}

template <int FMT, bool OB>
__global__ __launch_bounds__(64 * kGWaves) void gemm_lp_kernel(ProjParams p) {
  constexpr bool kFp4 = FMT == kFmtMxfp4;
  constexpr int kInstr = kFp4 ? 2 : 1;              // instructions per step
  constexpr int kRows = kGM + kGN;
  constexpr int kCodeBytes = kRows * 128;            // per buffer
  constexpr int kScaleBytes = kFp4 ? kRows * 8 : 0;  // per buffer
  constexpr int kSLoads = kFp4 ? kRows * 8 / 4 / 64 / kGWaves : 0;
  __shared__ __align__(16) uint8_t smem[kGStages][kCodeBytes + kScaleBytes];

  int64_t m0;
  int n0;
  tile_origin(p, m0, n0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // Code loads as in the bf16 kernel, over rows of rb code bytes.
  const int rb = kFp4 ? p.K / 2 : p.K;
  const char* xb = reinterpret_cast<const char*>(p.xq) + m0 * rb;
  const char* wb = static_cast<const char*>(p.w) + (int64_t)n0 * rb;
  uint32_t off[kGLoads];
#pragma unroll
  for (int i = 0; i < kGLoads; ++i) {
    const int cr = 8 * (kGWaves * i + wave) + (lane >> 3);
    const int q = (lane & 7) ^ ((cr >> 1) & 7);
    const int r = cr < kGM ? (int)min((int64_t)cr, p.M - 1 - m0)
                           : min(cr - kGM, p.N - 1 - n0);
    off[i] = (uint32_t)r * (uint32_t)rb + 16u * q;
  }
  // Scale loads (MXFP4): dword d = 64 (kGWaves u + w) + lane holds scales
  // 4 (d & 1) .. +3 of the step's 8 for combined row d >> 1; in LDS the
  // step's scales sit row after row, 8 bytes each.
  const int nblk = p.K / 32;
  const char* xsb = static_cast<const char*>(p.xs) + m0 * nblk;
  const char* wsb = static_cast<const char*>(p.wscale) + (int64_t)n0 * nblk;
  uint32_t soff[kSLoads > 0 ? kSLoads : 1];
#pragma unroll
  for (int u = 0; u < kSLoads; ++u) {
    const int d = 64 * (kGWaves * u + wave) + lane;
    const int cr = d >> 1;
    const int r = cr < kGM ? (int)min((int64_t)cr, p.M - 1 - m0)
                           : min(cr - kGM, p.N - 1 - n0);
    soff[u] = (uint32_t)r * (uint32_t)nblk + 4u * (d & 1);
  }
  const int steps = rb / 128;
  auto issue = [&](int s, int buf) {
    const int st = min(s, steps - 1);
#pragma unroll
    for (int i = 0; i < kGLoads; ++i)
      dma16((8 * kGWaves * i < kGM ? xb : wb) + st * 128 + off[i],
              &smem[buf][128 * 8 * (kGWaves * i + wave)]);
#pragma unroll
    for (int u = 0; u < kSLoads; ++u)
      dma4((64 * kGWaves * u < 2 * kGM ? xsb : wsb) + st * 8 + soff[u],
             &smem[buf][kCodeBytes + 256 * (kGWaves * u + wave)]);
  };
  // Wait for every load of the next step and this wave's LDS reads, then
  // for every wave's.
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(gwait(0));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto granule = [&](const uint8_t* base, int r, int q) {
    return *reinterpret_cast<const u32x4_t*>(base + 2 * gsw(r, q));
  };

  f32x4_t acc[8][kTJ];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < kTJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  issue(0, 0);
  sync();
  issue(1, 1);
  int cur = 0;
  if constexpr (!kFp4) {
    // FP8: one instruction per step, so the step splits by tokens instead of
    // K.  Half A (token tiles 0..3) runs while the fragments of half B are
    // read; after the barrier, half B runs weight tile by weight tile, and
    // each next-step weight fragment is read as soon as the last
    // instruction using its registers has issued, together with half A's
    // token fragments of the next step.
    static_assert(kTJ == 4, "half B reads one token tile per weight tile");
    i32x8_t xa[4], xb[4], w[kTJ];
    auto rd_x = [&](i32x8_t& dst, const uint8_t* sA, int i) {
      const int r = wm * 128 + 16 * i + c;
      const u32x4_t v0 = granule(sA, r, 2 * g), v1 = granule(sA, r, 2 * g + 1);
      dst = i32x8_t{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                    (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
    };
    auto rd_w = [&](int j, const uint8_t* sB) {
      const int r = wn * kWR + 16 * j + c;
      const u32x4_t v0 = granule(sB, r, 2 * g), v1 = granule(sB, r, 2 * g + 1);
      w[j] = i32x8_t{(int)v0[0], (int)v0[1], (int)v0[2], (int)v0[3],
                     (int)v1[0], (int)v1[1], (int)v1[2], (int)v1[3]};
    };
#pragma unroll
    for (int t = 0; t < 4; ++t) rd_x(xa[t], smem[0], t);
#pragma unroll
    for (int j = 0; j < kTJ; ++j) rd_w(j, smem[0] + kGM * 128);
    for (int s = 0; s < steps; ++s) {
      const uint8_t* sA = smem[cur];
      // The reads of xa and w were issued during the previous half B and
      // are done; saying so keeps the compiler from also waiting for xb.
      __builtin_amdgcn_s_waitcnt(kLdsDone);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        rd_x(xb[t], sA, 4 + t);
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
          acc[t][j] = mfma_scaled<0>(w[j], xa[t], acc[t][j], 127, 127);
      }
      sync();
      issue(s + 2, cur);
      cur ^= 1;
      const uint8_t* nA = smem[cur];
      const uint8_t* nB = smem[cur] + kGM * 128;
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[4 + t][j] = mfma_scaled<0>(w[j], xb[t], acc[4 + t][j], 127, 127);
        rd_w(j, nB);
        rd_x(xa[j], nA, j);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // MXFP4: two instructions per step (kc = 0, 1), each split into the same
    // token halves as FP8: half B of instruction 0 reads instruction 1's
    // fragments; half B of instruction 1 runs after the barrier and reads
    // the next step's instruction-0 fragments.  E2M1 operands take 4
    // registers (the upper half of the 8-register operand is zero).
    static_assert(kTJ == 4, "half B reads one token tile per weight tile");
    u32x4_t xa[4], xb[4], w[kTJ];
    int xsa[4], xsb[4], wsc[kTJ];
    auto rd_x = [&](u32x4_t& dst, int& sc, const uint8_t* buf, int i, int kc) {
      const int r = wm * 128 + 16 * i + c;
      dst = granule(buf, r, 4 * kc + g);
      sc = buf[kCodeBytes + 8 * r + 4 * kc + g];
    };
    auto rd_w = [&](int j, const uint8_t* buf, int kc) {
      const int r = wn * kWR + 16 * j + c;
      w[j] = granule(buf + kGM * 128, r, 4 * kc + g);
      wsc[j] = buf[kCodeBytes + 8 * (kGM + r) + 4 * kc + g];
    };
    auto op = [](const u32x4_t& v) {
      return i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
    };
    // Half A: token tiles 0..3 while half B's fragments of instruction kc
    // are read from buf.
    auto half_a = [&](const uint8_t* buf, int kc) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        rd_x(xb[t], xsb[t], buf, 4 + t, kc);
#pragma unroll
        for (int j = 0; j < kTJ; ++j)
          acc[t][j] = mfma_scaled<4>(op(w[j]), op(xa[t]), acc[t][j], wsc[j], xsa[t]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // Half B: token tiles 4..7 weight tile by weight tile, each freed weight
    // fragment (and a token tile of half A) refilled for instruction kc of
    // buf.
    auto half_b = [&](const uint8_t* buf, int kc) {
#pragma unroll
      for (int j = 0; j < kTJ; ++j) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[4 + t][j] = mfma_scaled<4>(op(w[j]), op(xb[t]), acc[4 + t][j], wsc[j], xsb[t]);
        rd_w(j, buf, kc);
        rd_x(xa[j], xsa[j], buf, j, kc);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int t = 0; t < 4; ++t) rd_x(xa[t], xsa[t], smem[0], t, 0);
#pragma unroll
    for (int j = 0; j < kTJ; ++j) rd_w(j, smem[0], 0);
    for (int s = 0; s < steps; ++s) {
      const uint8_t* b = smem[cur];
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      half_a(b, 0);
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      half_b(b, 1);
      __builtin_amdgcn_s_waitcnt(kLdsDone);
      half_a(b, 1);
      sync();
      issue(s + 2, cur);
      cur ^= 1;
      half_b(smem[cur], 0);
    }
  }
  // Drain the loads issued past the last step before the workgroup ends.
  __builtin_amdgcn_s_waitcnt(gwait(0));

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t m = m0 + wm * 128 + 16 * i + c;
    if (m >= p.M) continue;
    const float xsc = kFp4 ? 1.0f : static_cast<const float*>(p.xs)[m];
#pragma unroll
    for (int j = 0; j < kTJ; ++j) {
      const int n = n0 + wn * kWR + 16 * j + 4 * g;
      if (n >= p.N) continue;
      float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      if constexpr (!kFp4) {
        const float4 ws4 =
            *reinterpret_cast<const float4*>(static_cast<const float*>(p.wscale) + n);
        v.x *= xsc * ws4.x;
        v.y *= xsc * ws4.y;
        v.z *= xsc * ws4.z;
        v.w *= xsc * ws4.w;
      }
      store4(p.out, m * p.N + n, v, OB);
    }
  }
}
}  // namespace

hipError_t launch_gemm_bf16(const ProjParams& p, hipStream_t s) {
  const bool q4k = p.wfmt == kFmtQ4K && p.wd;
  if ((p.wfmt != kFmtBf16 && !q4k) || !p.x_bf16 || p.K % kBK != 0 ||
      (q4k ? 2 * (int64_t)p.K : p.K) > kGemmMaxK || p.splits != 1)
    return hipErrorInvalidValue;
  const int64_t tiles = ((p.M + kGM - 1) / kGM) * ((p.N + kGN - 1) / kGN);
  if (p.out_bf16) gemm_bf16_kernel<true><<<(unsigned)tiles, 64 * kGWaves, 0, s>>>(p);
  else gemm_bf16_kernel<false><<<(unsigned)tiles, 64 * kGWaves, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gemm_lp(const ProjParams& p, hipStream_t s) {
  const bool fp4 = p.wfmt == kFmtMxfp4;
  if ((p.wfmt != kFmtFp8 && !fp4) || p.K % (fp4 ? 256 : 128) != 0 ||
      p.K > kGemmMaxK || p.splits != 1)
    return hipErrorInvalidValue;
  const int64_t tiles = ((p.M + kGM - 1) / kGM) * ((p.N + kGN - 1) / kGN);
  const dim3 grid((unsigned)tiles), block(64 * kGWaves);
  if (fp4) {
    if (p.out_bf16) gemm_lp_kernel<kFmtMxfp4, true><<<grid, block, 0, s>>>(p);
    else gemm_lp_kernel<kFmtMxfp4, false><<<grid, block, 0, s>>>(p);
  } else {
    if (p.out_bf16) gemm_lp_kernel<kFmtFp8, true><<<grid, block, 0, s>>>(p);
    else gemm_lp_kernel<kFmtFp8, false><<<grid, block, 0, s>>>(p);
  }
  return hipGetLastError();
}

}  // namespace gdn
