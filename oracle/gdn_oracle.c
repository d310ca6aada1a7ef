/*
 * gdn_oracle.c -- plain fp64 CPU oracle for the gated delta-rule recurrent core
 * and its gated-RMSNorm tail.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; it exists so that tests, the smoke check and the CPU baseline leg
 * of the benchmark have an obviously-correct, independent reference.  It shares
 * no code, header, table or constant with the HIP library.
 *
 * What it follows (the pages, by title and section):
 *  - "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098),
 *    Abstract, mechanism (ii): the decay gate is a softplus/exponential
 *    parameterization and the write strength a sigmoid one; mechanism (iii):
 *    the delta-rule recurrence overwrites the state along the current key
 *    direction, and the fixed-size state summarizes the context.
 *  - "A Node-by-Node White-Box Walkthrough of a Quantized Hybrid Gated DeltaNet
 *    Language Model", Principais Resultados: the recurrent scan over the
 *    associative memory matrix S is the only route by which earlier tokens
 *    enter; forget gates form a fixed spectrum of time scales.
 *  - "Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection",
 *    section "Pinned graph semantics", steps 1-5: per 128-value head RMSNorm
 *    with one shared weight vector, times SiLU(z), flattened head-major.
 *
 * The exact update is the gated delta rule of the layer:
 *     S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,   o_t = S_t q_t
 * with S a d_v x d_k matrix (row i = value index i, contiguous over keys),
 *     a_t = exp(-exp(A_log) * softplus(g_t + dt_bias)),   b_t = sigmoid(beta_t).
 * The oracle evaluates it token by token, term by term:
 *     S_{t-1}(I - b k k^T) = S_{t-1} - b (S_{t-1} k) k^T,
 * so S_t = a S_{t-1} - a b (S_{t-1} k) k^T + b v k^T.  No chunking, blocking or
 * reordering.  Rows of S never interact (each row only meets k, q and its own
 * v entry), so the OpenMP loop runs over (sequence, value head, row block).
 *
 * Readings where the pages are silent (listed again in the design notes):
 *  - key head of value head h is h / (h_v / h_k) (consecutive value heads
 *    share a key head);
 *  - no 1/sqrt(d_k) query scaling, no in-oracle L2 normalisation;
 *  - the read-out uses the post-update state S_t;
 *  - softplus(x) = log(1 + e^x) exactly, no threshold; plain sigmoid;
 *  - tail: y = o * (mean(o^2) + eps)^(-1/2) * w * (z * sigmoid(z)).
 *
 * Every floating-point operation is double precision.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define GDN_ORACLE_GATES_RAW 0
#define GDN_ORACLE_GATES_DIRECT 1

/* softplus(x) = log(1 + exp(x)), written in the overflow-free form
   max(x, 0) + log1p(exp(-|x|)). */
static double oracle_softplus(double x) {
  return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

/* sigmoid(x) = 1 / (1 + exp(-x)). */
static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Decay a_t and write strength b_t of one (token, value head).
   Gated DeltaNet paper, Abstract (ii): softplus/exponential decay gate and
   sigmoid write gate.  RAW mode: g and beta are pre-activations, A_log and
   dt_bias the per-head parameters.  DIRECT mode: g already holds log a_t and
   beta already holds b_t. */
static void oracle_gate(int mode, double g, double beta, double A_log,
                        double dt_bias, double* a, double* b) {
  if (mode == GDN_ORACLE_GATES_DIRECT) {
    *a = exp(g);
    *b = beta;
  } else {
    *a = exp(-exp(A_log) * oracle_softplus(g + dt_bias));
    *b = oracle_sigmoid(beta);
  }
}

/* Exported for the gate pins: fills a[i], b[i] for n (g, beta) pairs of one
   head. */
void gdn_oracle_gates(int64_t n, int mode, const double* g, const double* beta,
                      double A_log, double dt_bias, double* a, double* b) {
  for (int64_t i = 0; i < n; ++i)
    oracle_gate(mode, g[i], beta[i], A_log, dt_bias, &a[i], &b[i]);
}

/* One token of the gated delta rule on n_rows consecutive value rows of one
   head (S points at the first of them, v and o at the matching entries):
     w_i   = S_i . k                       (the state read along the key)
     S_i  <- a S_i - a b w_i k^T + b v_i k^T
     o_i   = S_i . q                       (read-out from the updated state)
   S_i is row i of the d_v x d_k state, stored contiguously over keys. */
static void oracle_token_rows(double* S, int d_k, int n_rows, double a,
                              double b, const double* k, const double* q,
                              const double* v, double* o) {
  for (int i = 0; i < n_rows; ++i) {
    double* Si = S + (size_t)i * d_k;
    double w = 0.0;
    for (int j = 0; j < d_k; ++j) w += Si[j] * k[j];
    for (int j = 0; j < d_k; ++j)
      Si[j] = a * Si[j] - a * b * w * k[j] + b * v[i] * k[j];
    double oi = 0.0;
    for (int j = 0; j < d_k; ++j) oi += Si[j] * q[j];
    o[i] = oi;
  }
}

/* The prefill loop gives each task ORACLE_ROW_BLOCK value rows of one head;
   the task keeps those rows in a local buffer of up to ORACLE_MAX_DK keys. */
#define ORACLE_ROW_BLOCK 8
#define ORACLE_MAX_DK 256
static int oracle_row_block(int d_v) {
  return d_v < ORACLE_ROW_BLOCK ? d_v : ORACLE_ROW_BLOCK;
}

/* Token-by-token prefill over packed variable-length sequences.
   Layouts (all row-major, contiguous):
     cu_seqlens    [n_seqs+1] token offsets, non-decreasing, cu[0] = 0
     q, k          [T, h_k, d_k]
     v             [T, h_v, d_v]
     g, beta       [T, h_v]
     A_log,dt_bias [h_v]        (ignored in DIRECT mode)
     initial_state [n_seqs, h_v, d_v, d_k] or NULL (= zeros)
     final_state   same shape, or NULL (= not written)
     o             [T, h_v, d_v] recurrent output (before the tail)
   Returns 0, or -1 on a shape error. */
int gdn_oracle_prefill(int n_seqs, const int64_t* cu_seqlens, int h_k, int h_v,
                       int d_k, int d_v, int gate_mode, const double* q,
                       const double* k, const double* v, const double* g,
                       const double* beta, const double* A_log,
                       const double* dt_bias, const double* initial_state,
                       double* final_state, double* o, int n_threads) {
  if (n_seqs < 0 || h_k <= 0 || h_v <= 0 || h_v % h_k != 0 || d_k <= 0 ||
      d_v <= 0 || d_k > ORACLE_MAX_DK)
    return -1;
  const int group = h_v / h_k;
  const int rb = oracle_row_block(d_v);
  const int n_rb = (d_v + rb - 1) / rb;
  const int64_t tasks = (int64_t)n_seqs * h_v * n_rb;
  const size_t state_sz = (size_t)d_v * d_k;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t task = 0; task < tasks; ++task) {
    const int n = (int)(task / ((int64_t)h_v * n_rb));
    const int h = (int)((task / n_rb) % h_v);
    const int r0 = (int)(task % n_rb) * rb;
    const int r1 = r0 + rb < d_v ? r0 + rb : d_v;
    const int hk = h / group;
    double S[ORACLE_ROW_BLOCK * ORACLE_MAX_DK]; /* rows r0..r1-1 of the state */
    const double* S0 =
        initial_state ? initial_state + ((size_t)n * h_v + h) * state_sz : NULL;
    for (int i = r0; i < r1; ++i)
      for (int j = 0; j < d_k; ++j)
        S[(size_t)(i - r0) * d_k + j] = S0 ? S0[(size_t)i * d_k + j] : 0.0;
    for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
      double a, b;
      const double A = gate_mode == GDN_ORACLE_GATES_DIRECT ? 0.0 : A_log[h];
      const double D = gate_mode == GDN_ORACLE_GATES_DIRECT ? 0.0 : dt_bias[h];
      oracle_gate(gate_mode, g[t * h_v + h], beta[t * h_v + h], A, D, &a, &b);
      oracle_token_rows(S, d_k, r1 - r0, a, b, k + ((size_t)t * h_k + hk) * d_k,
                        q + ((size_t)t * h_k + hk) * d_k,
                        v + ((size_t)t * h_v + h) * d_v + r0,
                        o + ((size_t)t * h_v + h) * d_v + r0);
    }
    if (final_state) {
      double* SF = final_state + ((size_t)n * h_v + h) * state_sz;
      for (int i = r0; i < r1; ++i)
        for (int j = 0; j < d_k; ++j)
          SF[(size_t)i * d_k + j] = S[(size_t)(i - r0) * d_k + j];
    }
  }
  return 0;
}

/* One decode step: one new token for each of n independent sequences, the
   state updated in place.  Layouts: q, k [n, h_k, d_k]; v [n, h_v, d_v];
   g, beta [n, h_v]; state [n, h_v, d_v, d_k]; o [n, h_v, d_v]. */
int gdn_oracle_decode(int n, int h_k, int h_v, int d_k, int d_v, int gate_mode,
                      const double* q, const double* k, const double* v,
                      const double* g, const double* beta, const double* A_log,
                      const double* dt_bias, double* state, double* o,
                      int n_threads) {
  if (n < 0 || h_k <= 0 || h_v <= 0 || h_v % h_k != 0 || d_k <= 0 || d_v <= 0)
    return -1;
  const int group = h_v / h_k;
  const size_t state_sz = (size_t)d_v * d_k;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t task = 0; task < (int64_t)n * h_v; ++task) {
    const int s = (int)(task / h_v), h = (int)(task % h_v), hk = h / group;
    double a, b;
    const double A = gate_mode == GDN_ORACLE_GATES_DIRECT ? 0.0 : A_log[h];
    const double D = gate_mode == GDN_ORACLE_GATES_DIRECT ? 0.0 : dt_bias[h];
    oracle_gate(gate_mode, g[task], beta[task], A, D, &a, &b);
    oracle_token_rows(state + (size_t)task * state_sz, d_k, d_v, a, b,
                      k + ((size_t)s * h_k + hk) * d_k,
                      q + ((size_t)s * h_k + hk) * d_k,
                      v + (size_t)task * d_v, o + (size_t)task * d_v);
  }
  return 0;
}

/* Gated RMSNorm tail, "Pinned graph semantics" steps 2-5: each row of d
   values (one head of one token) is RMS-normalised with the shared weight w,
   then multiplied by SiLU(z) = z * sigmoid(z).  Rows are laid out head-major,
   so [T, h_v, d] rows flatten to [T, h_v * d] outputs without a copy. */
void gdn_oracle_gated_rmsnorm(int64_t rows, int d, const double* x,
                              const double* z, const double* w, double eps,
                              double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* xr = x + (size_t)r * d;
    const double* zr = z + (size_t)r * d;
    double* yr = out + (size_t)r * d;
    double ss = 0.0;
    for (int i = 0; i < d; ++i) ss += xr[i] * xr[i];
    const double inv_rms = 1.0 / sqrt(ss / d + eps);
    for (int i = 0; i < d; ++i) {
      const double normed = xr[i] * inv_rms * w[i];
      const double silu = zr[i] * oracle_sigmoid(zr[i]);
      yr[i] = normed * silu;
    }
  }
}

/* Number of threads OpenMP will use for the parallel loops above. */
int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
