// gdn_device.h -- device helpers shared by the gfx950 kernels of libgdn:
// bf16 <-> fp32 conversion, vector loads of either io dtype, cross-lane sums
// on 64-wide wavefronts, and the gate functions of the layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Native clang vectors (usable with the nontemporal builtins, unlike float4).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 ----
// bf16 is the top half of an fp32 bit pattern.  Widening is exact; narrowing
// rounds to nearest even, which gfx950 does in one instruction
// (v_cvt_pk_bf16_f32; a NaN stays a quiet NaN).
typedef __bf16 gdn_bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Packs two floats into one 32-bit word of two bf16 (lo first in memory).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const gdn_bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four consecutive elements starting at element index idx (a multiple of 4)
// of an fp32 (is_bf16 = false) or bf16 (is_bf16 = true) array.
__device__ __forceinline__ float4 load4(const void* base, int64_t idx,
                                        bool is_bf16) {
  if (is_bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(
        static_cast<const uint16_t*>(base) + idx);
    return make_float4(bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                       bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
}

__device__ __forceinline__ float load1(const void* base, int64_t idx,
                                       bool is_bf16) {
  if (is_bf16)
    return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  return static_cast<const float*>(base)[idx];
}

__device__ __forceinline__ void store4(void* base, int64_t idx, float4 v,
                                       bool is_bf16) {
  if (is_bf16) {
    uint2 w;
    w.x = pack_bf16x2(v.x, v.y);
    w.y = pack_bf16x2(v.z, v.w);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = v;
  }
}

__device__ __forceinline__ void store1(void* base, int64_t idx, float v,
                                       bool is_bf16) {
  if (is_bf16)
    static_cast<uint16_t*>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
  else
    static_cast<float*>(base)[idx] = v;
}

// ------------------------------------------------------- lane exchange ----
// DPP control words (data-parallel primitives inside a row of 16 lanes).
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,// lane i <-> 7 - i inside each half row
  kDppRowMirror = 0x140,    // lane i <-> 15 - i inside each row
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(
      0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N a power of two <= 64);
// every lane of the group receives the total.  Steps inside 16 lanes use DPP
// (no LDS traffic); the 16- and 32-lane steps use a cross-lane permute.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

// -------------------------------------------------------------- gates -----
// Decay and write strength of the layer ("Why Gated DeltaNet Survives 4-Bit
// Quantization", Abstract (ii): softplus/exponential decay, sigmoid write).
// log_decay returns log a = -exp(A_log) * softplus(g + dt_bias), the value the
// scans accumulate; DIRECT mode passes g through as log a and beta as b.
__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float log_decay_f32(float g, float A_log,
                                               float dt_bias, bool direct) {
  if (direct) return g;
  return -expf(A_log) * softplus_f32(g + dt_bias);
}

__device__ __forceinline__ float write_strength_f32(float beta, bool direct) {
  if (direct) return beta;
  return 1.0f / (1.0f + expf(-beta));
}

__device__ __forceinline__ double log_decay_f64(float g, float A_log,
                                                float dt_bias, bool direct) {
  if (direct) return (double)g;
  const double x = (double)g + (double)dt_bias;
  const double sp = fmax(x, 0.0) + log1p(exp(-fabs(x)));
  return -exp((double)A_log) * sp;
}

__device__ __forceinline__ double write_strength_f64(float beta, bool direct) {
  if (direct) return (double)beta;
  return 1.0 / (1.0 + exp(-(double)beta));
}

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + expf(-z));
}

// SiLU from the hardware base-2 exponential and reciprocal (each about one
// ulp): z * 1 / (1 + 2^(-z log2 e)).  Large negative z gives 2^(+big) = inf
// and a result of -0; large positive z gives z.  Relative error about 3e-7,
// for streaming kernels where the libm form would bound the throughput.
__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace gdn
