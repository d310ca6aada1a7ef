// rmsnorm.hip -- standalone gated RMSNorm (gfx950).
//
// "Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection", Pinned
// graph semantics steps 2-5: every head of d values is RMS-normalised with the
// shared weight vector, multiplied elementwise by SiLU(z), and the heads are
// laid out head-major, so rows of a [T, h_v, d] tensor map to a [T, h_v * d]
// output with no data movement:
//     out[r, i] = x[r, i] * rsqrt(mean_i x[r, :]^2 + eps) * w[i] * SiLU(z[r, i]).
//
// Memory-bound.  Each lane owns 4 consecutive values of a row; LPR = d / 4
// lanes share a row and sum their squares with DPP/permute steps; a wave
// covers 64 / LPR rows per pass and waves stride over the rows.  Every lane
// reads its values once and writes them once, so out may alias x.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kRmsThreads = 256;

template <int D>
__global__ __launch_bounds__(kRmsThreads) void rmsnorm_kernel(RmsParams p) {
  constexpr int LPR = D / 4;
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = (lane % LPR) * 4;
  const int rsub = lane / LPR;
  const float4 w4 = *reinterpret_cast<const float4*>(p.w + col);
  const int64_t waves_total = (int64_t)gridDim.x * (kRmsThreads / 64);
  for (int64_t rg = (int64_t)blockIdx.x * (kRmsThreads / 64) + wave;
       rg * RPW < p.rows; rg += waves_total) {
    const int64_t r = rg * RPW + rsub;
    const bool ok = r < p.rows;
    float4 x4 = make_float4(0.f, 0.f, 0.f, 0.f), z4 = x4;
    if (ok) {
      x4 = load4(p.x, r * D + col, p.x_bf16 != 0);
      z4 = load4(p.z, r * D + col, p.z_bf16 != 0);
    }
    float ss = x4.x * x4.x + x4.y * x4.y + x4.z * x4.z + x4.w * x4.w;
    ss = group_sum<LPR>(ss);
    const float inv = rsqrtf(ss / (float)D + p.eps);
    if (ok) {
      float4 y;
      y.x = x4.x * inv * w4.x * silu_f32(z4.x);
      y.y = x4.y * inv * w4.y * silu_f32(z4.y);
      y.z = x4.z * inv * w4.z * silu_f32(z4.z);
      y.w = x4.w * inv * w4.w * silu_f32(z4.w);
      store4(p.out, r * D + col, y, p.out_bf16 != 0);
    }
  }
}

template <int D>
hipError_t launch_d(const RmsParams& p, hipStream_t stream) {
  constexpr int RPW = 64 / (D / 4);
  const int64_t rows_per_block = (int64_t)RPW * (kRmsThreads / 64);
  int64_t blocks = (p.rows + rows_per_block - 1) / rows_per_block;
  const int64_t cap = 256 * 16;  // enough waves to keep every CU streaming
  if (blocks > cap) blocks = cap;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((rmsnorm_kernel<D>), dim3((unsigned)blocks),
                     dim3(kRmsThreads), 0, stream, p);
  return hipGetLastError();
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
