// gdn_proj.h -- parameter block, plan and launcher of the output projection
// kernels (proj.hip, gemm.hip), shared with the C-ABI front end (gdn_api.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Weight formats (same values as the C ABI's GDN_WEIGHT_*).
enum : int32_t { kFmtBf16 = 0, kFmtQ4K = 1, kFmtFp8 = 2, kFmtMxfp4 = 3 };

struct ProjParams {
  const void* x;          // [M, K] x dtype
  const void* w;          // bf16 [N, K]; Q4_K blocks [N, K / 256]; E4M3
                          // codes [N, K]; or packed E2M1 codes [N, K / 2]
  const void* wscale;     // FP8: fp32 [N]; MXFP4: E8M0 [N, K / 32]
  void* out;              // [M, N] out dtype
  float* ws;              // split-K partial sums [splits, M, N], or NULL
  uint8_t* xq;            // FP8 / MXFP4: quantized x codes (workspace)
  void* xs;               // FP8: fp32 [M] scales; MXFP4: E8M0 [M, K / 32]
  uint16_t* wd;           // Q4_K above 4096 tokens: W decoded into bf16
                          // parts, row n = [K high parts | K low parts]
                          // (workspace), or NULL
  int64_t M;
  int32_t K, N;
  int32_t x_bf16, out_bf16, wfmt;
  int32_t splits;         // K ranges (1 = no split)
};

// Kernel and K split the projection uses for given sizes; shared by the
// workspace query and the launch.  The workspace holds, in order, the
// quantized activations (FP8 / MXFP4 weights only), their scales, and the
// split-K slabs, or (Q4_K against bf16 activations above 4096 tokens) the
// decoded weight; each part starts 256-byte aligned.
enum class ProjKernel { kGemv, kTile32x64, kTile64x64, kTile128x128, kGemm };
struct ProjPlan {
  ProjKernel kernel;
  int32_t splits;
  size_t ws_bytes;
  size_t xq_off, xs_off, slab_off, wd_off;
};
ProjPlan plan_out_proj(int64_t M, int32_t K, int32_t N, int32_t wfmt,
                       bool x_f32);

// Activation quantization for the FP8 / MXFP4 projections (also exposed on
// its own): x [M, K] -> codes and scales as described for ProjParams.
struct QuantParams {
  const void* x;
  uint8_t* codes;
  void* scales;
  int64_t M;
  int32_t K;
  int32_t x_bf16, fmt;    // fmt: kFmtFp8 or kFmtMxfp4
};
hipError_t launch_quantize(const QuantParams& q, hipStream_t stream);

hipError_t launch_out_proj(const ProjParams& p, hipStream_t stream);

// 256 x 256 tile GEMMs with direct-to-LDS loads (gemm.hip), for many tokens.
// K at most kGemmMaxK (a lane's load offsets within a 256-row tile are
// 32-bit), no K split; hipErrorInvalidValue otherwise.  launch_gemm_bf16:
// dense bf16 weight and activations, K a multiple of 64, or the decoded
// Q4_K weight in wd (its rows 2 K long, x walked twice).  launch_gemm_lp:
// FP8 or MXFP4 weight codes against the quantized activations in xq / xs,
// K a multiple of 128 (FP8) or 256 (MXFP4).
constexpr int32_t kGemmMaxK = 1 << 22;
hipError_t launch_gemm_bf16(const ProjParams& p, hipStream_t stream);
hipError_t launch_gemm_lp(const ProjParams& p, hipStream_t stream);

}  // namespace gdn
