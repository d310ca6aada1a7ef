// decode.hip -- decode steps of the gated delta rule with the gated-RMSNorm
// tail fused in (gfx950): T tokens of each of N independent sequences per
// call, T = 1 being the plain decode step.
//
// The layer ("Why Gated DeltaNet Survives 4-Bit Quantization", Abstract (iii);
// "Red Lite dev15d", Pinned graph semantics): for each sequence n and value
// head h, with key head hk = h / (h_v / h_k), token after token,
//     S <- a S (I - b k k^T) + b v k^T,   o = S q,
// then optionally y = o * rsqrt(mean(o^2) + eps) * w * SiLU(z).
// Row i of S (a value index) evolves on its own:
//     u_i = S_i . k,  p_i = S_i . q,  delta_i = b (v_i - a u_i),
//     S_i <- a S_i + delta_i k^T,   o_i = a p_i + (k . q) delta_i.
// So a step is one pass over the fp32 state: every row is reduced against k
// and q and updated.
//
// Mapping: one workgroup per (sequence, value head), owning all d_v rows so
// the tail needs no cross-workgroup exchange.  Inside a wave, LPR consecutive
// lanes share a row: each lane holds NL float4 of it, and one wave-wide load
// instruction covers RPI rows x 4*LPR contiguous floats (whole 128-byte
// lines).  The state of the (sequence, head) stays in registers for all T
// tokens: it is read from HBM once before the first token and written once,
// row by row as the last token updates it, so a call costs one state round
// trip however many tokens
// it carries (the multi-token form serves speculative verification of draft
// tokens: "Nanbeige4.2-3B-NVFP4-FP8-LoopShield", Speed; "A Node-by-Node
// White-Box Walkthrough of a Quantized Hybrid Gated DeltaNet LM", open
// problems).  With snapshots requested, the state after every token is also
// written, so a caller can resume from the last accepted token.  All loads
// of a wave are issued before any reduction; the row sums use DPP inside
// groups of LPR <= 8 lanes, so every lane of the group receives u_i, p_i and
// updates its own columns with no broadcast.  State traffic is nontemporal:
// 512 MiB at the batched-decode size, larger than the last-level cache.
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
  const bool direct = p.direct != 0;
  const float A_log = direct ? 0.f : p.A_log[h];
  const float dt_bias = direct ? 0.f : p.dt_bias[h];

  float* S = p.state + (int64_t)nh * DV * DK;
  const int row0 = wave * RW + rl;

  // Inputs of one token for this lane: gates, its columns of k and q, and
  // v at its rows.  Token ti+1's are fetched while token ti is processed;
  // token 0's before the state, so they do not queue behind it.
  struct TokIn {
    float g, beta;
    float4 k4[NL], q4[NL];
    float v[G];
    float z;   // z of output element (threadIdx.x mod d_v), with the tail
  };
  auto load_tok = [&](int ti, TokIn& in) {
    const int64_t tok = (int64_t)n * p.T + ti;
    const int64_t th = tok * p.h_v + h;
    in.g = p.g[th];
    in.beta = p.beta[th];
    const int64_t kq_base = (tok * p.h_k + hk) * DK;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
      const int col = (m * LPR + cl) * 4;
      in.k4[m] = load4(p.k, kq_base + col, io16);
      in.q4[m] = load4(p.q, kq_base + col, io16);
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
      in.v[gi] = load1(p.v, th * DV + row0 + gi * RPI, io16);
    in.z = p.tail ? load1(p.z, th * DV + (threadIdx.x & (DV - 1)), io16) : 0.f;
  };
  TokIn cur;
  load_tok(0, cur);

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

  const int t = threadIdx.x;
  for (int ti = 0; ti < p.T; ++ti) {
    const int64_t tok = (int64_t)n * p.T + ti;   // row of this token's inputs
    const int64_t th = tok * p.h_v + h;
    TokIn nxt;
    if (ti + 1 < p.T) load_tok(ti + 1, nxt);

    // Gates of this (token, value head).
    const float la = log_decay_f32(cur.g, A_log, dt_bias, direct);
    const float a = expf(la);
    const float b = write_strength_f32(cur.beta, direct);
    const float4* k4 = cur.k4;
    const float4* q4 = cur.q4;
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < NL; ++m)
      kq += k4[m].x * q4[m].x + k4[m].y * q4[m].y + k4[m].z * q4[m].z +
            k4[m].w * q4[m].w;
    kq = group_sum<LPR>(kq);

    const int64_t v_base = th * DV;
    float* snap = p.snaps ? p.snaps + th * DV * DK : nullptr;
    // The last token streams each updated row straight back to the state
    // (in place), as a single step does; earlier tokens keep it in registers.
    const bool last = ti == p.T - 1;
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
      const float delta = b * (cur.v[gi] - a * u);
      const float o = a * pq + kq * delta;
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        s[gi][m].x = a * s[gi][m].x + delta * k4[m].x;
        s[gi][m].y = a * s[gi][m].y + delta * k4[m].y;
        s[gi][m].z = a * s[gi][m].z + delta * k4[m].z;
        s[gi][m].w = a * s[gi][m].w + delta * k4[m].w;
        if (snap)
          __builtin_nontemporal_store(
              s[gi][m], reinterpret_cast<f32x4*>(snap + (int64_t)r * DK) + m * LPR + cl);
        if (last)
          __builtin_nontemporal_store(
              s[gi][m], reinterpret_cast<f32x4*>(S + (int64_t)r * DK) + m * LPR + cl);
      }
      if (cl == 0) o_lds[r] = o;
    }
    __syncthreads();

    if (!p.tail) {
      if (t < DV) store1(p.out, v_base + t, o_lds[t], p.out_bf16 != 0);
    } else {
      // Fused gated RMSNorm of this head (d_v values).
      if (wave == 0) {
        float ss = 0.f;
        for (int i = lane; i < DV; i += 64) ss += o_lds[i] * o_lds[i];
        ss = group_sum<64>(ss);
        if (lane == 0) red_lds = rsqrtf(ss / (float)DV + p.eps);
      }
      __syncthreads();
      if (t < DV) {
        const float y = o_lds[t] * red_lds * p.w[t] * silu_f32(cur.z);
        store1(p.out, v_base + t, y, p.out_bf16 != 0);
      }
    }
    __syncthreads();   // o_lds and red_lds are reused by the next token
    if (ti + 1 < p.T) cur = nxt;
  }

}

template <int DK, int DV>
hipError_t launch_dkdv(const DecodeParams& p, hipStream_t stream) {
  using Sh = DecodeShape<DK, DV>;
  const int blocks = p.N * p.h_v;
  if (blocks == 0 || p.T == 0) return hipSuccess;
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
