// decode.hip -- one decode step of the gated delta rule with the gated-RMSNorm
// tail fused in (gfx950).
//
// The layer ("Why Gated DeltaNet Survives 4-Bit Quantization", Abstract (iii);
// "Red Lite dev15d", Pinned graph semantics): for each sequence n and value
// head h, with key head hk = h / (h_v / h_k),
//     S <- a S (I - b k k^T) + b v k^T,   o = S q,
// then optionally y = o * rsqrt(mean(o^2) + eps) * w * SiLU(z).
// Row i of S (a value index) evolves on its own:
//     u_i = S_i . k,  p_i = S_i . q,  delta_i = b (v_i - a u_i),
//     S_i <- a S_i + delta_i k^T,   o_i = a p_i + (k . q) delta_i.
// So the step is one streaming pass over the fp32 state: every row is read
// once, reduced against k and q, updated and written back in place.
//
// Mapping: one workgroup per (sequence, value head), owning all d_v rows so
// the tail needs no cross-workgroup exchange.  Inside a wave, LPR consecutive
// lanes share a row: each lane holds NL float4 of it, and one wave-wide load
// instruction covers RPI rows x 4*LPR contiguous floats (whole 128-byte
// lines).  All loads of a wave are issued before any reduction so that
// 16 x 16 bytes per lane are in flight.  The row sums use DPP inside groups
// of LPR <= 8 lanes, so every lane of the group receives u_i, p_i and can
// update its own columns with no broadcast.  The state is streamed with
// nontemporal loads and stores: 512 MiB at the batched-decode size is read
// once and written once, larger than the last-level cache.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

template <int DK, int DV>
struct DecodeShape {
  static constexpr int LPR = DK >= 32 ? 8 : 4;          // lanes per row
  static constexpr int NL = DK / (4 * LPR);              // float4 per lane/row
  static constexpr int RPI = 64 / LPR;                   // rows per wave load
  static constexpr int W0 = DV / RPI;
  static constexpr int WAVES = W0 < 1 ? 1 : (W0 > 4 ? 4 : W0);
  static constexpr int RW = DV / WAVES;                  // rows per wave
  static constexpr int G = RW / RPI;                     // row groups per wave
  static constexpr int THREADS = WAVES * 64;
  static_assert(DK % (4 * LPR) == 0, "d_k");
  static_assert(RW % RPI == 0 && G >= 1, "d_v");
};

template <int DK, int DV>
__global__ __launch_bounds__((DecodeShape<DK, DV>::THREADS))
void decode_kernel(DecodeParams p) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int LPR = Sh::LPR, NL = Sh::NL, RPI = Sh::RPI, RW = Sh::RW;
  constexpr int G = Sh::G;
  __shared__ float o_lds[DV];
  __shared__ float red_lds;

  const int nh = blockIdx.x;                 // n * h_v + h
  const int n = nh / p.h_v;
  const int h = nh - n * p.h_v;
  const int hk = h / p.group;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rl = lane / LPR;                 // row inside a load group
  const int cl = lane % LPR;                 // column lane inside the row
  const bool io16 = p.io_bf16 != 0;

  // Gates of this (token, value head).
  const float gv = p.g[nh], bv = p.beta[nh];
  const bool direct = p.direct != 0;
  const float la = log_decay_f32(gv, direct ? 0.f : p.A_log[h],
                                 direct ? 0.f : p.dt_bias[h], direct);
  const float a = expf(la);
  const float b = write_strength_f32(bv, direct);

  // This lane's columns of k and q.
  const int64_t kq_base = ((int64_t)n * p.h_k + hk) * DK;
  float4 k4[NL], q4[NL];
  float kq = 0.f;
#pragma unroll
  for (int m = 0; m < NL; ++m) {
    const int col = (m * LPR + cl) * 4;
    k4[m] = load4(p.k, kq_base + col, io16);
    q4[m] = load4(p.q, kq_base + col, io16);
    kq += k4[m].x * q4[m].x + k4[m].y * q4[m].y + k4[m].z * q4[m].z +
          k4[m].w * q4[m].w;
  }
  kq = group_sum<LPR>(kq);

  float* S = p.state + (int64_t)nh * DV * DK;
  const int row0 = wave * RW + rl;

  // Stream in every row this lane touches.
  f32x4 s[G][NL];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int r = row0 + gi * RPI;
#pragma unroll
    for (int m = 0; m < NL; ++m)
      s[gi][m] = __builtin_nontemporal_load(
          reinterpret_cast<const f32x4*>(S + (int64_t)r * DK) + m * LPR + cl);
  }

  const int64_t v_base = (int64_t)nh * DV;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int r = row0 + gi * RPI;
    float u = 0.f, pq = 0.f;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      u += s[gi][m].x * k4[m].x + s[gi][m].y * k4[m].y + s[gi][m].z * k4[m].z +
           s[gi][m].w * k4[m].w;
      pq += s[gi][m].x * q4[m].x + s[gi][m].y * q4[m].y +
            s[gi][m].z * q4[m].z + s[gi][m].w * q4[m].w;
    }
    u = group_sum<LPR>(u);
    pq = group_sum<LPR>(pq);
    const float vr = load1(p.v, v_base + r, io16);
    const float delta = b * (vr - a * u);
    const float o = a * pq + kq * delta;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      f32x4 t;
      t.x = a * s[gi][m].x + delta * k4[m].x;
      t.y = a * s[gi][m].y + delta * k4[m].y;
      t.z = a * s[gi][m].z + delta * k4[m].z;
      t.w = a * s[gi][m].w + delta * k4[m].w;
      __builtin_nontemporal_store(
          t, reinterpret_cast<f32x4*>(S + (int64_t)r * DK) + m * LPR + cl);
    }
    if (cl == 0) o_lds[r] = o;
  }
  __syncthreads();

  const int t = threadIdx.x;
  if (!p.tail) {
    if (t < DV) store1(p.out, v_base + t, o_lds[t], p.out_bf16 != 0);
    return;
  }
  // Fused gated RMSNorm of this head (d_v values).
  if (wave == 0) {
    float ss = 0.f;
    for (int i = lane; i < DV; i += 64) ss += o_lds[i] * o_lds[i];
    ss = group_sum<64>(ss);
    if (lane == 0) red_lds = rsqrtf(ss / (float)DV + p.eps);
  }
  __syncthreads();
  if (t < DV) {
    const float zt = load1(p.z, v_base + t, io16);
    const float y = o_lds[t] * red_lds * p.w[t] * silu_f32(zt);
    store1(p.out, v_base + t, y, p.out_bf16 != 0);
  }
}

template <int DK, int DV>
hipError_t launch_dkdv(const DecodeParams& p, hipStream_t stream) {
  using Sh = DecodeShape<DK, DV>;
  const int blocks = p.N * p.h_v;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_kernel<DK, DV>), dim3(blocks), dim3(Sh::THREADS),
                     0, stream, p);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_dk(const DecodeParams& p, hipStream_t stream) {
  switch (p.d_v) {
    case 16: return launch_dkdv<DK, 16>(p, stream);
    case 32: return launch_dkdv<DK, 32>(p, stream);
    case 64: return launch_dkdv<DK, 64>(p, stream);
    case 128: return launch_dkdv<DK, 128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  switch (p.d_k) {
    case 16: return launch_dk<16>(p, stream);
    case 32: return launch_dk<32>(p, stream);
    case 64: return launch_dk<64>(p, stream);
    case 128: return launch_dk<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
