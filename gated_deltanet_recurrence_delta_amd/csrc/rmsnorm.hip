// rmsnorm.hip -- standalone gated RMSNorm (gfx950).
//
// "Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection", Pinned
// graph semantics steps 2-5: every head of d values is RMS-normalised with the
// shared weight vector, multiplied elementwise by SiLU(z), and the heads are
// laid out head-major, so rows of a [T, h_v, d] tensor map to a [T, h_v * d]
// output with no data movement:
//     out[r, i] = x[r, i] * rsqrt(mean_i x[r, :]^2 + eps) * w[i] * SiLU(z[r, i]).
//
// Memory-bound.  Each lane owns 8 consecutive values of a row; LPR = d / 8
// lanes share a row and sum their squares with DPP steps (permute for the
// widest rows); a wave covers 64 / LPR rows per step and keeps kUnroll such
// steps in flight, with every load issued before the first use, so that
// enough bytes are outstanding to stream at HBM rate.  Loads and stores are
// nontemporal: each value is touched once.  Every lane reads its values once
// and writes exactly those values, so out may alias x.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRmsThreads = 256;
constexpr int kUnroll = 4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Eight consecutive values at element idx (a multiple of 8) of an fp32 or
// bf16 array.
template <bool BF16>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + idx));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const f32x4* p4 = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    const f32x4 a = __builtin_nontemporal_load(p4);
    const f32x4 b = __builtin_nontemporal_load(p4 + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

template <bool BF16>
__device__ __forceinline__ void store8(void* base, int64_t idx, const float (&v)[8]) {
  if constexpr (BF16) {
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    __builtin_nontemporal_store(
        w, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(base) + idx));
  } else {
    f32x4* p4 = reinterpret_cast<f32x4*>(static_cast<float*>(base) + idx);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, p4);
    __builtin_nontemporal_store(f32x4{v[4], v[5], v[6], v[7]}, p4 + 1);
  }
}

template <int D, bool XB, bool ZB, bool OB>
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_kernel(RmsParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * 8;
  const int rsub = lane / LPR;
  float w8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w8[i] = p.w[col + i];
  const int64_t groups = (p.rows + RPW - 1) / RPW;
  const int64_t waves_total = (int64_t)gridDim.x * (kRmsThreads / 64);
  for (int64_t g0 = (int64_t)blockIdx.x * (kRmsThreads / 64) + wave; g0 < groups;
       g0 += waves_total * kUnroll) {
    float x[kUnroll][8], z[kUnroll][8];
    int64_t r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      r[u] = (g0 + u * waves_total) * RPW + rsub;
      // Rows past the end load the last row (no branch around the loads);
      // their results are not stored.
      const int64_t rc = r[u] < p.rows ? r[u] : p.rows - 1;
      load8<XB>(p.x, rc * D + col, x[u]);
      load8<ZB>(p.z, rc * D + col, z[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += x[u][i] * x[u][i];
      ss = group_sum<LPR>(ss);
      const float inv = rsqrtf(ss / (float)D + p.eps);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = x[u][i] * inv * w8[i] * silu_f32(z[u][i]);
      if (r[u] < p.rows) store8<OB>(p.out, r[u] * D + col, y);
    }
  }
}

template <int D, bool XB, bool ZB, bool OB>
hipError_t launch_t(const RmsParams& p, hipStream_t stream) {
  constexpr int RPW = 64 / (D / 8);
  const int64_t rows_per_block = (int64_t)RPW * (kRmsThreads / 64) * kUnroll;
  int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 8;  // 8 workgroups per compute unit
  if (blocks > cap) blocks = cap;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rmsnorm_kernel<D, XB, ZB, OB>), dim3((unsigned)blocks),
                     dim3(kRmsThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const RmsParams& p, hipStream_t stream) {
  const int sel = (p.x_bf16 ? 4 : 0) | (p.z_bf16 ? 2 : 0) | (p.out_bf16 ? 1 : 0);
  switch (sel) {
    case 0: return launch_t<D, false, false, false>(p, stream);
    case 1: return launch_t<D, false, false, true>(p, stream);
    case 2: return launch_t<D, false, true, false>(p, stream);
    case 3: return launch_t<D, false, true, true>(p, stream);
    case 4: return launch_t<D, true, false, false>(p, stream);
    case 5: return launch_t<D, true, false, true>(p, stream);
    case 6: return launch_t<D, true, true, false>(p, stream);
    default: return launch_t<D, true, true, true>(p, stream);
  }
}

}  // namespace

hipError_t launch_rmsnorm(const RmsParams& p, hipStream_t stream) {
  switch (p.d) {
    case 16: return launch_d<16>(p, stream);
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
    case 256: return launch_d<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
