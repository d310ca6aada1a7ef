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
// The inputs of up to 8 tokens (gates, k, q, v, z) are loaded together and
// staged in LDS, the next batch's while the current one runs; since rows
// are independent, the tokens of a batch follow one another with no barrier,
// their read-outs collected in LDS, and one barrier later each wave
// normalises and stores the outputs of its share of the batch's tokens.
// Calls with several tokens per sequence run decode_tokens_kernel, the same
// pass with row groups outer and tokens inner (see there).
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// Tokens whose inputs the multi-token kernel stages in LDS at a time.
constexpr int kTokenBatch = 8;

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
  constexpr int G = Sh::G, WAVES = Sh::WAVES, THREADS = Sh::THREADS;
  // Tokens whose inputs are staged in LDS at a time.
  constexpr int TB = 8;
  __shared__ float k_l[TB][DK], q_l[TB][DK], v_l[TB][DV], z_l[TB][DV];
  __shared__ float o_l[TB][DV];
  __shared__ float g_l[TB], b_l[TB];

  const int nh = blockIdx.x;                 // n * h_v + h
  const int n = nh / p.h_v;
  const int h = nh - n * p.h_v;
  const int hk = h / p.group;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int rl = lane / LPR;                 // row inside a load group
  const int cl = lane % LPR;                 // column lane inside the row
  const bool io16 = p.io_bf16 != 0;
  const bool direct = p.direct != 0;
  const float A_log = direct ? 0.f : p.A_log[h];
  const float dt_bias = direct ? 0.f : p.dt_bias[h];

  float* S = p.state + (int64_t)nh * DV * DK;
  const int row0 = wave * RW + rl;

  // The inputs of tokens b0 .. b0 + nb - 1 (gates, k, q, v and z rows of
  // this head) into registers; every load of the batch is issued before any
  // is used, so a batch costs one memory latency rather than one per token.
  constexpr int NK4 = (TB * DK / 4 + THREADS - 1) / THREADS;
  constexpr int NV4 = (TB * DV / 4 + THREADS - 1) / THREADS;
  float4 kr[NK4], qr[NK4], vr[NV4], zr[NV4];
  float gr = 0.f, br = 0.f;
  auto fetch = [&](int b0, int nb) {
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DK, col = e % DK;
      if (ti < nb) {
        const int64_t base = (((int64_t)n * p.T + b0 + ti) * p.h_k + hk) * DK + col;
        kr[i] = load4(p.k, base, io16);
        qr[i] = load4(p.q, base, io16);
      }
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DV, col = e % DV;
      if (ti < nb) {
        const int64_t base = (((int64_t)n * p.T + b0 + ti) * p.h_v + h) * DV + col;
        vr[i] = load4(p.v, base, io16);
        if (p.tail) zr[i] = load4(p.z, base, io16);
      }
    }
    if (t < nb) {
      const int64_t th = ((int64_t)n * p.T + b0 + t) * p.h_v + h;
      gr = p.g[th];
      br = p.beta[th];
    }
  };
  auto stage = [&](int nb) {
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DK, col = e % DK;
      if (ti < nb) {
        *reinterpret_cast<float4*>(&k_l[ti][col]) = kr[i];
        *reinterpret_cast<float4*>(&q_l[ti][col]) = qr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DV, col = e % DV;
      if (ti < nb) {
        *reinterpret_cast<float4*>(&v_l[ti][col]) = vr[i];
        if (p.tail) *reinterpret_cast<float4*>(&z_l[ti][col]) = zr[i];
      }
    }
    if (t < nb) {
      g_l[t] = gr;
      b_l[t] = br;
    }
  };

  // Token 0's batch first, so that it does not queue behind the state.
  fetch(0, p.T < TB ? p.T : TB);
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

  for (int b0 = 0; b0 < p.T; b0 += TB) {
    const int nb = p.T - b0 < TB ? p.T - b0 : TB;
    stage(nb);
    __syncthreads();
    // The next batch's inputs load while this one is processed.
    if (b0 + TB < p.T) fetch(b0 + TB, p.T - b0 - TB < TB ? p.T - b0 - TB : TB);

    // The state chain: rows are independent, so tokens follow one another
    // with no barrier; each token's read-out goes to LDS for the tail.
    for (int ti = 0; ti < nb; ++ti) {
      const int64_t th = ((int64_t)n * p.T + b0 + ti) * p.h_v + h;
      const float la = log_decay_f32(g_l[ti], A_log, dt_bias, direct);
      const float a = expf(la);
      const float b = write_strength_f32(b_l[ti], direct);
      float4 k4[NL], q4[NL];
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        k4[m] = *reinterpret_cast<const float4*>(&k_l[ti][(m * LPR + cl) * 4]);
        q4[m] = *reinterpret_cast<const float4*>(&q_l[ti][(m * LPR + cl) * 4]);
      }
      float kq = 0.f;
#pragma unroll
      for (int m = 0; m < NL; ++m)
        kq += k4[m].x * q4[m].x + k4[m].y * q4[m].y + k4[m].z * q4[m].z +
              k4[m].w * q4[m].w;
      kq = group_sum<LPR>(kq);

      float* snap = p.snaps ? p.snaps + th * DV * DK : nullptr;
      // The last token streams each updated row straight back to the state
      // (in place), as a single step does; earlier tokens keep it in
      // registers.
      const bool last = b0 + ti == p.T - 1;
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
        const float delta = b * (v_l[ti][r] - a * u);
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
        if (cl == 0) o_l[ti][r] = o;
      }
    }
    __syncthreads();

    // Outputs of the batch: wave w takes tokens w, w + WAVES, ...
    for (int ti = wave; ti < nb; ti += WAVES) {
      const int64_t v_base = (((int64_t)n * p.T + b0 + ti) * p.h_v + h) * DV;
      if (!p.tail) {
        for (int i = lane; i < DV; i += 64) store1(p.out, v_base + i, o_l[ti][i], p.out_bf16 != 0);
      } else {
        // Fused gated RMSNorm of this head (d_v values).
        float ss = 0.f;
        for (int i = lane; i < DV; i += 64) ss += o_l[ti][i] * o_l[ti][i];
        ss = group_sum<64>(ss);
        const float inv = rsqrtf(ss / (float)DV + p.eps);
        for (int i = lane; i < DV; i += 64) {
          const float y = o_l[ti][i] * inv * p.w[i] * silu_f32(z_l[ti][i]);
          store1(p.out, v_base + i, y, p.out_bf16 != 0);
        }
      }
    }
    __syncthreads();   // the batch's LDS is reused by the next one
  }
}

// Several tokens per sequence: the same pass with the loops exchanged --
// each row group of a wave runs all of a batch's tokens before the next
// group, so a group waits only for its own state loads and streams its rows
// back while the later groups still compute, and workgroups do not all
// stall on their token work at once.  The input dtype is a template
// parameter and every load of a batch is unconditional, so the loads carry
// no branch and issue back to back, and no wait for the inputs waits for the
// state.  NEXT (calls of more than one batch) compiles in the prefetch of the
// next batch; a call of one batch has nothing to prefetch.  (For one token
// the plain kernel above is faster.)
template <int DK, int DV, bool IO16, bool NEXT>
__global__ __launch_bounds__((DecodeShape<DK, DV>::THREADS))
void decode_tokens_kernel(DecodeParams p) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int LPR = Sh::LPR, NL = Sh::NL, RPI = Sh::RPI, RW = Sh::RW;
  constexpr int G = Sh::G, WAVES = Sh::WAVES, THREADS = Sh::THREADS;
  // Tokens whose inputs are staged in LDS at a time.
  constexpr int TB = kTokenBatch;
  __shared__ float k_l[TB][DK], q_l[TB][DK], v_l[TB][DV], z_l[TB][DV];
  __shared__ float o_l[TB][DV];
  __shared__ float g_l[TB], b_l[TB];
  __shared__ float a_l[TB], bb_l[TB], kq_l[TB];   // a, b and k . q of each token

  const int nh = blockIdx.x;                 // n * h_v + h
  const int n = nh / p.h_v;
  const int h = nh - n * p.h_v;
  const int hk = h / p.group;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int rl = lane / LPR;                 // row inside a load group
  const int cl = lane % LPR;                 // column lane inside the row
  constexpr bool io16 = IO16;
  const bool direct = p.direct != 0;
  const float A_log = direct ? 0.f : p.A_log[h];
  const float dt_bias = direct ? 0.f : p.dt_bias[h];

  float* S = p.state + (int64_t)nh * DV * DK;
  const int row0 = wave * RW + rl;

  // The inputs of tokens b0 .. b0 + nb - 1 (gates, k, q, v and z rows of
  // this head) into registers; every load of the batch is issued before any
  // is used, so a batch costs one memory latency rather than one per token.
  // The loads are unconditional (slots past the batch reload its first
  // token, and without a tail z reloads v), so the compiler counts them
  // exactly and later waits need not wait for the state.
  constexpr int NK4 = (TB * DK / 4 + THREADS - 1) / THREADS;
  constexpr int NV4 = (TB * DV / 4 + THREADS - 1) / THREADS;
  float4 kr[NK4], qr[NK4], vr[NV4], zr[NV4];
  float gr = 0.f, br = 0.f;
  auto fetch = [&](int b0, int nb) {
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DK, col = e % DK;
      const int tc = ti < nb ? ti : 0;
      const int64_t base = (((int64_t)n * p.T + b0 + tc) * p.h_k + hk) * DK + col;
      kr[i] = load4(p.k, base, io16);
      qr[i] = load4(p.q, base, io16);
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DV, col = e % DV;
      const int tc = ti < nb ? ti : 0;
      const int64_t base = (((int64_t)n * p.T + b0 + tc) * p.h_v + h) * DV + col;
      vr[i] = load4(p.v, base, io16);
      zr[i] = load4(p.tail ? p.z : p.v, base, io16);
    }
    {
      const int tc = t < nb ? t : 0;
      const int64_t th = ((int64_t)n * p.T + b0 + tc) * p.h_v + h;
      gr = p.g[th];
      br = p.beta[th];
    }
  };
  // Every staged value is written (rows past the batch hold its first
  // token again and are never read), so no load waits inside a branch.
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DK, col = e % DK;
      if (ti < TB) {
        *reinterpret_cast<float4*>(&k_l[ti][col]) = kr[i];
        *reinterpret_cast<float4*>(&q_l[ti][col]) = qr[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (t + i * THREADS) * 4, ti = e / DV, col = e % DV;
      if (ti < TB) {
        *reinterpret_cast<float4*>(&v_l[ti][col]) = vr[i];
        *reinterpret_cast<float4*>(&z_l[ti][col]) = zr[i];
      }
    }
    if (t < TB) {
      g_l[t] = gr;
      b_l[t] = br;
    }
  };

  // Token 0's batch first, so that it does not queue behind the state.
  fetch(0, p.T < TB ? p.T : TB);
  __builtin_amdgcn_sched_barrier(0);
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

  // One batch of tokens; the first is peeled off the loop, so that the
  // state registers its loads write are the ones its row groups use (a
  // loop-carried copy would wait for every load first).
  auto run_batch = [&](int b0) {
    const int nb = p.T - b0 < TB ? p.T - b0 : TB;
    stage();
    __syncthreads();
    // The next batch's inputs load while this one is processed (after the
    // last batch, the last batch's again: the loads stay unconditional, so
    // the compiler's count of loads in flight stays exact).
    if constexpr (NEXT) {
      const int b1 = b0 + TB < p.T ? b0 + TB : b0;
      fetch(b1, p.T - b1 < TB ? p.T - b1 : TB);
    }

    // Per-token scalars of the batch (a, b and k . q), one wave per token.
    for (int ti = wave; ti < nb; ti += WAVES) {
      float kq = 0.f;
#pragma unroll
      for (int m = 0; m < NL; ++m) {
        const float4 k4 = *reinterpret_cast<const float4*>(&k_l[ti][(m * LPR + cl) * 4]);
        const float4 q4 = *reinterpret_cast<const float4*>(&q_l[ti][(m * LPR + cl) * 4]);
        kq += k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w;
      }
      kq = group_sum<LPR>(kq);
      if (lane == 0) {
        a_l[ti] = expf(log_decay_f32(g_l[ti], A_log, dt_bias, direct));
        bb_l[ti] = write_strength_f32(b_l[ti], direct);
        kq_l[ti] = kq;
      }
    }
    __syncthreads();

    // The state chain.  Rows are independent, so each row group runs all
    // the batch's tokens before the next group starts: a group needs only
    // its own loads to have arrived, and after the last token it streams
    // its rows back while the later groups still compute.  Each token's
    // read-out goes to LDS for the tail.
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int r = row0 + gi * RPI;
      for (int ti = 0; ti < nb; ++ti) {
        const int64_t th = ((int64_t)n * p.T + b0 + ti) * p.h_v + h;
        const float a = a_l[ti], b = bb_l[ti], kq = kq_l[ti];
        float4 k4[NL], q4[NL];
#pragma unroll
        for (int m = 0; m < NL; ++m) {
          k4[m] = *reinterpret_cast<const float4*>(&k_l[ti][(m * LPR + cl) * 4]);
          q4[m] = *reinterpret_cast<const float4*>(&q_l[ti][(m * LPR + cl) * 4]);
        }
        float* snap = p.snaps ? p.snaps + th * DV * DK : nullptr;
        // The last token streams each updated row straight back to the
        // state (in place), as a single step does; earlier tokens keep it in
        // registers.
        const bool last = b0 + ti == p.T - 1;
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
        const float delta = b * (v_l[ti][r] - a * u);
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
        if (cl == 0) o_l[ti][r] = o;
      }
    }
    __syncthreads();

    // Outputs of the batch: wave w takes tokens w, w + WAVES, ...
    for (int ti = wave; ti < nb; ti += WAVES) {
      const int64_t v_base = (((int64_t)n * p.T + b0 + ti) * p.h_v + h) * DV;
      if (!p.tail) {
        for (int i = lane; i < DV; i += 64) store1(p.out, v_base + i, o_l[ti][i], p.out_bf16 != 0);
      } else {
        // Fused gated RMSNorm of this head (d_v values).
        float ss = 0.f;
        for (int i = lane; i < DV; i += 64) ss += o_l[ti][i] * o_l[ti][i];
        ss = group_sum<64>(ss);
        const float inv = rsqrtf(ss / (float)DV + p.eps);
        for (int i = lane; i < DV; i += 64) {
          const float y = o_l[ti][i] * inv * p.w[i] * silu_f32(z_l[ti][i]);
          store1(p.out, v_base + i, y, p.out_bf16 != 0);
        }
      }
    }
    __syncthreads();   // the batch's LDS is reused by the next one
  };
  run_batch(0);
  for (int b0 = TB; b0 < p.T; b0 += TB) run_batch(b0);
}

template <int DK, int DV>
hipError_t launch_dkdv(const DecodeParams& p, hipStream_t stream) {
  using Sh = DecodeShape<DK, DV>;
  const int blocks = p.N * p.h_v;
  if (blocks == 0 || p.T == 0) return hipSuccess;
  if (p.T == 1)
    hipLaunchKernelGGL((decode_kernel<DK, DV>), dim3(blocks), dim3(Sh::THREADS),
                       0, stream, p);
  else if (p.T > kTokenBatch) {   // several batches: prefetch the next one
    if (p.io_bf16)
      hipLaunchKernelGGL((decode_tokens_kernel<DK, DV, true, true>), dim3(blocks),
                         dim3(Sh::THREADS), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_tokens_kernel<DK, DV, false, true>), dim3(blocks),
                         dim3(Sh::THREADS), 0, stream, p);
  } else if (p.io_bf16) {
    hipLaunchKernelGGL((decode_tokens_kernel<DK, DV, true, false>), dim3(blocks),
                       dim3(Sh::THREADS), 0, stream, p);
  } else {
    hipLaunchKernelGGL((decode_tokens_kernel<DK, DV, false, false>), dim3(blocks),
                       dim3(Sh::THREADS), 0, stream, p);
  }
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
