// gdn_proj.h -- parameter block, plan and launcher of the output projection
// kernels (proj.hip), shared with the C-ABI front end (gdn_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ProjParams {
  const void* x;          // [M, K] x dtype
  const void* w;          // dense bf16 [N, K], or Q4_K blocks [N, K / 256]
  void* out;              // [M, N] out dtype
  float* ws;              // split-K partial sums [splits, M, N], or NULL
  int64_t M;
  int32_t K, N;
  int32_t x_bf16, out_bf16, q4k;
  int32_t splits;         // K ranges (1 = no split)
};

// Kernel and K split the projection uses for given sizes; shared by the
// workspace query and the launch.
enum class ProjKernel { kGemv, kTile32x64, kTile64x64, kTile128x128 };
struct ProjPlan {
  ProjKernel kernel;
  int32_t splits;
  size_t ws_bytes;
};
ProjPlan plan_out_proj(int64_t M, int32_t K, int32_t N, bool q4k,
                       bool x_f32);

hipError_t launch_out_proj(const ProjParams& p, hipStream_t stream);

}  // namespace gdn
