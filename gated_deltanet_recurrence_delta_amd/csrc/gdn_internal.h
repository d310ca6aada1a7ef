// gdn_internal.h -- parameter blocks and launchers shared between the C-ABI
// front end (gdn_api.hip) and the kernel translation units.  Host code only
// passes plain pointers and sizes; every launcher enqueues on `stream` and
// returns the HIP launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  const float* s0;        // may be NULL (zeros)
  float* sF;              // may be NULL (not written)
  const void* z;          // NULL: no tail
  const float* w;
  void* out;
  const int32_t* cu;      // device offsets, or NULL (equal lengths)
  float* ws;              // workspace (fp32), may be NULL
  int64_t T;
  int32_t N;
  int32_t seq_len;        // T / N when cu == NULL
  int32_t h_k, h_v, group;
  int32_t d_k, d_v, chunk;
  int32_t io_bf16, out_bf16, direct, tail;
  int32_t slices;         // value-row slices per (sequence, value head)
  float eps;
};

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* A_log;
  const float* dt_bias;
  float* state;
  float* snaps;           // state after every token, or NULL
  const void* z;
  const float* w;
  void* out;
  int32_t N, T;           // sequences, tokens per sequence
  int32_t h_k, h_v, group, d_k, d_v;
  int32_t io_bf16, out_bf16, direct, tail;
  float eps;
};

struct RmsParams {
  const void* x;
  const void* z;
  const float* w;
  void* out;
  int64_t rows;
  int32_t d;
  int32_t x_bf16, z_bf16, out_bf16;
  float eps;
};

struct PrologueParams {
  const void* x;          // [T, C] io dtype: q | k | v channels
  const float* w;         // [C, W]
  const float* bias;      // [C] or NULL
  const int32_t* cu;      // device offsets [N+1], or NULL (one sequence)
  const float* s0;        // [N, C, W-1] or NULL (zeros)
  float* sF;              // [N, C, W-1] or NULL
  void* q;                // [T, h_k, d_k] out dtype
  void* k;
  void* v;                // [T, h_v, d_v]
  int64_t T, C;
  int32_t N, h_k, h_v, d_k, d_v, W;
  int32_t io_bf16, out_bf16;
  float eps;
};

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
hipError_t launch_prologue(const PrologueParams& p, hipStream_t stream);
hipError_t launch_rmsnorm(const RmsParams& p, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, hipStream_t stream);

// Whether the library selects the bf16 MFMA prefill for these shapes.
extern const bool kHaveBf16Mfma;

// Work split of the bf16 MFMA prefill for given sizes (value-row slices per
// head and workspace bytes); used both by the workspace query and the launch.
struct Bf16Plan {
  int32_t slices;
  size_t ws_bytes;
};
Bf16Plan plan_prefill_bf16(int64_t T, int32_t N, int32_t h_k, int32_t h_v,
                           int32_t d_v, bool tail);

}  // namespace gdn
