// prefill_f32.hip -- chunked prefill of the gated delta rule computed in fp32
// on the vector ALUs (gfx950).  The general-purpose path: fp32 or bf16 inputs,
// d_k = d_v = D in {16, 32, 64, 128}, chunk C in {16, 32, 64}, packed
// sequences, carried state, shared key heads and the fused gated-RMSNorm tail.
//
// Per (sequence, value head) the scan walks the sequence in chunks of C
// tokens (chunks restart at each sequence start; the last may be short and is
// zero-padded, which leaves the state untouched: k = 0, b = 0, log a = 0).
// With S0 the state entering the chunk, ell = log a, G = chunk-local prefix
// sum of ell (kept in fp64: the cumulative decay spans hundreds of nats at the
// strongest gates), E_ij = exp(G_i - G_j) on j <= i:
//     A = strict_lower(diag(b) (E o K K^T)),    P = E o Q K^T   (j <= i)
//     R = diag(b) (V - diag(e^G) K S0^T)
//     U = (I + A)^{-1} R        (forward substitution: the UT transform)
//     O = diag(e^G) Q S0^T + P U
//     S = e^{G_L} S0 + (diag(e^{G_L - G}) U)^T K
// which equals the token-by-token rule in exact arithmetic.
//
// Mapping: one 256-thread workgroup per (sequence, value head).  The state
// lives in registers: thread t owns row i = t / TPR and the columns
// j = (t % TPR) + TPR * m of it, TPR = 256 / D.  Token columns of R, U (in
// LDS `U`) and O (in LDS `O`) are indexed [token][row]; a row's TPR lanes
// split every token sum among themselves (lane p takes tokens = p mod TPR)
// and combine with a DPP group sum.  In the substitution the lane that writes
// U[c][i] is the one that later reads it back, so the sequential loop over
// tokens needs no barrier.  A and P share one C x C tile: P on and below the
// diagonal, A transposed above it.
#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_seqmap.h"

namespace gdn {
namespace {

constexpr int kF32Threads = 256;

template <int D, int C>
struct F32Lds {
  float K[C][D + 1];
  float Q[C][D + 1];
  float U[C][D + 1];    // V -> R -> U, token-major
  float O[C][D + 1];    // diag(e^G) Q S0^T -> O
  float AP[C][C + 1];   // P[i][j] at [i][j] (j <= i); A[i][j] at [j][i] (j < i)
  double G[C];
  float eG[C];          // e^{G_c}
  float eGL[C];         // e^{G_L - G_c}
  float b[C];
  float inv_rms[C];
};

template <int D, int C>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(
    PrefillParams p) {
  constexpr int TPR = kF32Threads / D;  // threads per state row
  constexpr int CPT = D / TPR;          // columns per thread
  __shared__ F32Lds<D, C> sm;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int row = t / TPR;
  const int part = t % TPR;
  const int nh = blockIdx.x;
  const int n = nh / p.h_v;
  const int h = nh - n * p.h_v;
  const int hk = h / p.group;
  const bool io16 = p.io_bf16 != 0;
  const bool direct = p.direct != 0;
  const float A_log = direct ? 0.f : p.A_log[h];
  const float dt_bias = direct ? 0.f : p.dt_bias[h];

  int64_t t_beg, t_end;
  seq_bounds(p.cu, n, p.seq_len, p.T, t_beg, t_end);

  const int64_t st_off = (int64_t)nh * D * D + (int64_t)row * D;
  float S[CPT];
#pragma unroll
  for (int m = 0; m < CPT; ++m)
    S[m] = p.s0 ? p.s0[st_off + part + TPR * m] : 0.f;

  for (int64_t c0 = t_beg; c0 < t_end; c0 += C) {
    const int L = (int)((t_end - c0) < C ? (t_end - c0) : C);
    __syncthreads();  // previous chunk is done with the LDS tiles
    // Stage K, Q (key head hk) and V (value head h); zero-pad past L.
    for (int e = t; e < C * (D / 4); e += kF32Threads) {
      const int c = e / (D / 4), j = (e % (D / 4)) * 4;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), qq = kk, vv = kk;
      if (c < L) {
        const int64_t tok = c0 + c;
        kk = load4(p.k, (tok * p.h_k + hk) * D + j, io16);
        qq = load4(p.q, (tok * p.h_k + hk) * D + j, io16);
        vv = load4(p.v, (tok * p.h_v + h) * D + j, io16);
      }
      sm.K[c][j] = kk.x; sm.K[c][j + 1] = kk.y; sm.K[c][j + 2] = kk.z; sm.K[c][j + 3] = kk.w;
      sm.Q[c][j] = qq.x; sm.Q[c][j + 1] = qq.y; sm.Q[c][j + 2] = qq.z; sm.Q[c][j + 3] = qq.w;
      sm.U[c][j] = vv.x; sm.U[c][j + 1] = vv.y; sm.U[c][j + 2] = vv.z; sm.U[c][j + 3] = vv.w;
    }
    // Gates and the chunk-local fp64 prefix sum of log a.
    if (wave == 0) {
      double ell = 0.0;
      float bb = 0.f;
      if (lane < L) {
        const int64_t gi = (c0 + lane) * p.h_v + h;
        ell = log_decay_f64(p.g[gi], A_log, dt_bias, direct);
        bb = (float)write_strength_f64(p.beta[gi], direct);
      }
      double G = ell;  // inclusive scan over the 64 lanes (C <= 64)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double o = __shfl_up(G, off, 64);
        if (lane >= off) G += o;
      }
      const double GL = __shfl(G, C - 1, 64);
      if (lane < C) {
        sm.G[lane] = G;
        sm.b[lane] = bb;
        sm.eG[lane] = (float)exp(G);
        sm.eGL[lane] = (float)exp(GL - G);
      }
    }
    __syncthreads();
    // A and P.
    for (int e = t; e < C * C; e += kF32Threads) {
      const int ci = e / C, cj = e % C;
      if (cj > ci) continue;
      float kk = 0.f, qk = 0.f;
      for (int j = 0; j < D; ++j) {
        const float kj = sm.K[cj][j];
        kk += sm.K[ci][j] * kj;
        qk += sm.Q[ci][j] * kj;
      }
      const float E = (float)exp(sm.G[ci] - sm.G[cj]);
      sm.AP[ci][cj] = E * qk;
      if (cj < ci) sm.AP[cj][ci] = sm.b[ci] * E * kk;
    }
    // R = diag(b)(V - diag(e^G) K S0^T) and diag(e^G) Q S0^T, per token.
    for (int c = 0; c < C; ++c) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int m = 0; m < CPT; ++m) {
        x += sm.K[c][part + TPR * m] * S[m];
        y += sm.Q[c][part + TPR * m] * S[m];
      }
      x = group_sum<TPR>(x);
      y = group_sum<TPR>(y);
      if (part == 0) {
        sm.U[c][row] = sm.b[c] * (sm.U[c][row] - sm.eG[c] * x);
        sm.O[c][row] = sm.eG[c] * y;
      }
    }
    __syncthreads();
    // U = (I + A)^{-1} R by forward substitution over the tokens.
    for (int c = 1; c < C; ++c) {
      float acc = 0.f;
      for (int cj = part; cj < c; cj += TPR) acc += sm.AP[cj][c] * sm.U[cj][row];
      acc = group_sum<TPR>(acc);
      const float u = sm.U[c][row] - acc;
      if (part == (c % TPR)) sm.U[c][row] = u;
    }
    __syncthreads();
    // O += P U, and S = e^{G_L} S0 + (diag(e^{G_L - G}) U)^T K.
    for (int c = 0; c < C; ++c) {
      float acc = 0.f;
      for (int cj = part; cj <= c; cj += TPR) acc += sm.AP[c][cj] * sm.U[cj][row];
      acc = group_sum<TPR>(acc);
      if (part == 0) sm.O[c][row] += acc;
    }
    const float eGL_all = sm.eG[C - 1];
#pragma unroll
    for (int m = 0; m < CPT; ++m) S[m] *= eGL_all;
    for (int c = 0; c < C; ++c) {
      const float uc = sm.eGL[c] * sm.U[c][row];
#pragma unroll
      for (int m = 0; m < CPT; ++m) S[m] += uc * sm.K[c][part + TPR * m];
    }
    __syncthreads();
    if (p.tail) {
      for (int c = wave; c < L; c += kF32Threads / 64) {
        float ss = 0.f;
        for (int i = lane; i < D; i += 64) ss += sm.O[c][i] * sm.O[c][i];
        ss = group_sum<64>(ss);
        if (lane == 0) sm.inv_rms[c] = rsqrtf(ss / (float)D + p.eps);
      }
      __syncthreads();
      for (int e = t; e < L * D; e += kF32Threads) {
        const int c = e / D, i = e % D;
        const int64_t oi = ((c0 + c) * p.h_v + h) * D + i;
        const float zz = load1(p.z, oi, io16);
        store1(p.out, oi, sm.O[c][i] * sm.inv_rms[c] * p.w[i] * silu_f32(zz),
               p.out_bf16 != 0);
      }
    } else {
      for (int e = t; e < L * D; e += kF32Threads) {
        const int c = e / D, i = e % D;
        store1(p.out, ((c0 + c) * p.h_v + h) * D + i, sm.O[c][i],
               p.out_bf16 != 0);
      }
    }
  }
  if (p.sF) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) p.sF[st_off + part + TPR * m] = S[m];
  }
}

template <int D, int C>
hipError_t launch_dc(const PrefillParams& p, hipStream_t stream) {
  const int blocks = p.N * p.h_v;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_f32_kernel<D, C>), dim3(blocks),
                     dim3(kF32Threads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillParams& p, hipStream_t stream) {
  switch (p.chunk) {
    case 16: return launch_dc<D, 16>(p, stream);
    case 32: return launch_dc<D, 32>(p, stream);
    case 64: return launch_dc<D, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillParams& p, hipStream_t stream) {
  switch (p.d_k) {
    case 16: return launch_d<16>(p, stream);
    case 32: return launch_d<32>(p, stream);
    case 64: return launch_d<64>(p, stream);
    case 128: return launch_d<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
