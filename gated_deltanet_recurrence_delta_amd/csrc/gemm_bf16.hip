// gemm_bf16.hip -- dense bf16 output projection for long prefills:
// y[m, :] = W x[m, :] with W [N out rows, K] and x [M, K] both bf16, fp32
// accumulation ("Red Lite dev15d -- DeltaNet gated tail + Q4_K output
// projection", Pinned graph semantics step 6, with the weight kept dense).
//
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

// s_waitcnt immediate: at most n vector memory operations outstanding and
// no LDS operation (vmcnt bits [3:0] and [15:14], lgkmcnt 0, expcnt not
// waited for).
constexpr int gwait(int n) { return ((n >> 4) << 14) | 0x0070 | (n & 15); }
// s_waitcnt immediate: no LDS operation outstanding (vmcnt and expcnt at
// their maxima, i.e. not waited for).
constexpr int kLdsDone = (3 << 14) | 0x0070 | 15;

template <bool OB>
__global__ __launch_bounds__(64 * kGWaves) void gemm_bf16_kernel(ProjParams p) {
  __shared__ __align__(16) uint16_t smem[kGStages][(kGM + kGN) * kBK];

  // Tile order as in the projection's tile kernels: each XCD takes a contiguous run of
  // tile ids, grouped 8 token panels at a time.
  const int tiles_m = (int)((p.M + kGM - 1) / kGM);
  const int tiles_n = (p.N + kGN - 1) / kGN;
  const int nb = gridDim.x, b = blockIdx.x;
  const int t = (nb % 8 == 0) ? (b & 7) * (nb >> 3) + (b >> 3) : b;
  constexpr int kGroup = 8;
  const int grp = t / (kGroup * tiles_n), in = t % (kGroup * tiles_n);
  const int gm = min(kGroup, tiles_m - grp * kGroup);
  const int64_t m0 = (int64_t)(grp * kGroup + in % gm) * kGM;
  const int n0 = (in / gm) * kGN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int wm = wave / kWavesN, wn = wave % kWavesN;

  // Sources of this lane's loads: load i of wave w covers rows
  // 8 (4 i + w) .. +7 of the combined tile (x rows 0..255, then W rows),
  // as a byte offset from the tile's first x or W row (a wave-uniform base,
  // so the load forms the address itself); rows past M or N repeat the last
  // one (valid addresses, never stored).
  const char* xb = static_cast<const char*>(p.x) + m0 * p.K * 2;
  const char* wb = static_cast<const char*>(p.w) + (int64_t)n0 * p.K * 2;
  uint32_t off[kGLoads];
#pragma unroll
  for (int i = 0; i < kGLoads; ++i) {
    const int cr = 8 * (kGWaves * i + wave) + (lane >> 3);
    const int q = (lane & 7) ^ ((cr >> 1) & 7);
    const int r = cr < kGM ? (int)min((int64_t)cr, p.M - 1 - m0)
                           : min(cr - kGM, p.N - 1 - n0);
    off[i] = (uint32_t)r * (uint32_t)p.K * 2u + 16u * q;
  }
  const int steps = p.K / kBK;
  auto issue = [&](int s, int buf) {
    const int k0 = min(s, steps - 1) * kBK * 2;
#pragma unroll
    for (int i = 0; i < kGLoads; ++i)
      __builtin_amdgcn_global_load_lds((8 * kGWaves * i < kGM ? xb : wb) + k0 + off[i],
                                       lds_addr(&smem[buf][8 * (kGWaves * i + wave) * kBK]),
                                       16, 0, 0);
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

}  // namespace

hipError_t launch_gemm_bf16(const ProjParams& p, hipStream_t s) {
  if (p.wfmt != kFmtBf16 || !p.x_bf16 || p.K % kBK != 0 || p.K > kGemmBf16MaxK ||
      p.splits != 1)
    return hipErrorInvalidValue;
  const int64_t tiles = ((p.M + kGM - 1) / kGM) * ((p.N + kGN - 1) / kGN);
  if (p.out_bf16) gemm_bf16_kernel<true><<<(unsigned)tiles, 64 * kGWaves, 0, s>>>(p);
  else gemm_bf16_kernel<false><<<(unsigned)tiles, 64 * kGWaves, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace gdn
