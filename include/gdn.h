/*
 * gdn.h -- C ABI of libgdn.so: the gated delta-rule recurrent core of a hybrid
 * LLM layer and its gated-RMSNorm tail, as hand-written HIP kernels for
 * MI355X (gfx950).
 *
 * The operation (pages by title and section):
 *  - "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098),
 *    Abstract: a Gated DeltaNet layer keeps a fixed-size recurrent state that
 *    summarizes the context (opening sentence); its decay and write-strength
 *    gates are softplus/exponential and sigmoid parameterizations (ii); the
 *    delta-rule recurrence overwrites the state along the current key
 *    direction (iii).  The update this library computes for every (sequence,
 *    value head), token by token in exact arithmetic, is
 *        S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t,
 *        a_t = exp(-exp(A_log) * softplus(g_t + dt_bias)),  b_t = sigmoid(beta_t),
 *    with S a d_v x d_k fp32 matrix (row i = value index i).
 *  - "A Node-by-Node White-Box Walkthrough of a Quantized Hybrid Gated
 *    DeltaNet Language Model", Principais Resultados: the recurrent scan over
 *    the associative memory matrix S is the only path by which earlier tokens
 *    enter the layer.
 *  - "Red Lite dev15d -- DeltaNet gated tail + Q4_K output projection",
 *    "Pinned graph semantics" steps 1-5 and "Real layer-0 GGUF tensors": the
 *    recurrent output and Z are viewed as value heads x 128, each head is
 *    RMS-normalised with one shared F32 weight of 128 values, multiplied by
 *    SiLU(z), and flattened head-major (32 x 128 -> 4096).
 *
 * Conventions shared by every entry point:
 *  - All tensors are dense, contiguous, row-major.  Tensor pointers are
 *    DEVICE pointers except the argument structs themselves and
 *    cu_seqlens_host.  The caller owns every buffer; the library allocates
 *    nothing at run time and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are enqueued asynchronously on it; the library never synchronizes.
 *  - Every call validates its arguments on the host before launching.  On
 *    any error nothing is launched, no output is touched, and a gdn_status
 *    code other than GDN_OK is returned.  No exception crosses the ABI.
 *  - Data-dependent conditions the host cannot see (device cu_seqlens
 *    contents, NaNs, DIRECT-mode gates outside their range) are the caller's
 *    responsibility; the kernels never read or write outside the sizes
 *    passed here: device offsets are clamped into [0, T] (for the prefill,
 *    each into [previous offset, T]) before use, so malformed offsets give
 *    wrong sequence boundaries, never an out-of-bounds access.
 *  - The library holds no mutable global state (apart from the scratch of
 *    gdn_chunk_prefill_noalloc, see there): calls on different streams may
 *    run concurrently as long as their output buffers are disjoint.
 *  - Key-head sharing: value head h reads key head h / (h_v / h_k).
 *  - No 1/sqrt(d_k) scaling and no normalisation of q or k is applied.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6u

/* Return codes. */
enum {
  GDN_OK = 0,
  GDN_E_NULL = 1,        /* a required pointer is NULL */
  GDN_E_SHAPE = 2,       /* a size is negative/zero or sizes disagree */
  GDN_E_DTYPE = 3,       /* unknown dtype or gate-mode value */
  GDN_E_UNSUPPORTED = 4, /* valid request the library has no kernel for */
  GDN_E_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  GDN_E_WORKSPACE = 6,   /* workspace missing or smaller than required */
  GDN_E_HIP = 7,         /* the HIP runtime reported an error */
  GDN_E_STRUCT = 8,      /* struct_size does not match this library */
  GDN_E_ALIAS = 9,       /* an output overlaps an input it must not */
  GDN_E_SCRATCH = 10     /* the call needs more workspace than the static
                            scratch of gdn_chunk_prefill_noalloc */
};

/* Element types. */
enum { GDN_F32 = 0, GDN_BF16 = 1 };

/* How g and beta are interpreted.
   RAW:    g, beta are pre-activations; a = exp(-exp(A_log[h]) *
           softplus(g + dt_bias[h])), b = sigmoid(beta).
   DIRECT: g holds log a (finite, <= 0) and beta holds b in [0, 1];
           A_log and dt_bias are ignored and may be NULL. */
enum { GDN_GATES_RAW = 0, GDN_GATES_DIRECT = 1 };

/* Chunked prefill over packed variable-length sequences. */
typedef struct gdn_prefill_args {
  uint32_t struct_size;          /* = sizeof(gdn_prefill_args) */
  int32_t num_seqs;              /* N >= 1 */
  int64_t total_tokens;          /* T >= 0, number of packed tokens */
  const int32_t* cu_seqlens;     /* device int32 [N+1]: token offsets with
                                    cu[0] = 0, non-decreasing, cu[N] = T.
                                    NULL: N sequences of T/N tokens each
                                    (T % N must be 0). Zero-length sequences
                                    are allowed (final = initial). */
  const int32_t* cu_seqlens_host;/* optional host copy of cu_seqlens, checked
                                    when given (starts at 0, non-decreasing,
                                    ends at T; without cu_seqlens it must be
                                    the even split).  The kernels take their
                                    boundaries from cu_seqlens.  May be NULL. */
  int32_t h_k, h_v;              /* key heads, value heads; h_v % h_k == 0 */
  int32_t d_k, d_v;              /* head sizes */
  int32_t chunk;                 /* chunk length C of the WY/UT scan */
  int32_t io_dtype;              /* dtype of q, k, v, z */
  int32_t out_dtype;             /* dtype of out */
  int32_t gate_mode;             /* GDN_GATES_RAW or GDN_GATES_DIRECT */
  const void* q;                 /* [T, h_k, d_k] */
  const void* k;                 /* [T, h_k, d_k] */
  const void* v;                 /* [T, h_v, d_v] */
  const float* g;                /* [T, h_v] fp32 */
  const float* beta;             /* [T, h_v] fp32 */
  const float* A_log;            /* [h_v] fp32 (RAW mode) */
  const float* dt_bias;          /* [h_v] fp32 (RAW mode) */
  const float* initial_state;    /* [N, h_v, d_v, d_k] fp32, NULL = zeros */
  float* final_state;            /* [N, h_v, d_v, d_k] fp32, NULL = not
                                    written; may equal initial_state */
  const void* z;                 /* [T, h_v, d_v] io dtype, or NULL */
  const float* norm_weight;      /* [d_v] fp32, required when z != NULL */
  float eps;                     /* RMSNorm epsilon (inside the root) */
  void* out;                     /* z == NULL: o [T, h_v, d_v];
                                    z != NULL: SiLU(z)-gated RMSNorm of o,
                                    flattened [T, h_v * d_v].
                                    Must not overlap any input. */
} gdn_prefill_args;

/* One decode step: one token for each of N independent sequences. */
typedef struct gdn_decode_args {
  uint32_t struct_size;          /* = sizeof(gdn_decode_args) */
  int32_t num_seqs;              /* N >= 0 */
  int32_t h_k, h_v, d_k, d_v;
  int32_t io_dtype, out_dtype, gate_mode;
  const void* q;                 /* [N, h_k, d_k] */
  const void* k;                 /* [N, h_k, d_k] */
  const void* v;                 /* [N, h_v, d_v] */
  const float* g;                /* [N, h_v] */
  const float* beta;             /* [N, h_v] */
  const float* A_log;            /* [h_v] (RAW mode) */
  const float* dt_bias;          /* [h_v] (RAW mode) */
  float* state;                  /* [N, h_v, d_v, d_k] fp32, read and updated
                                    in place */
  const void* z;                 /* [N, h_v, d_v] io dtype, or NULL */
  const float* norm_weight;      /* [d_v], required when z != NULL */
  float eps;
  void* out;                     /* o [N, h_v, d_v] or gated [N, h_v * d_v] */
} gdn_decode_args;

/* Several decode tokens per sequence in one call: tokens_per_seq = T
   consecutive tokens of each of N independent sequences, e.g. to verify T
   draft tokens of speculative decoding ("Nanbeige4.2-3B-NVFP4-FP8-LoopShield",
   Speed: decode served with a speculative verify batch; "A Node-by-Node
   White-Box Walkthrough of a Quantized Hybrid Gated DeltaNet LM", open
   problems: draft acceptance).  Token t of sequence n reads row n*T + t of
   q, k, v, z, g, beta and writes row n*T + t of out; the rule is applied
   token after token exactly as in gdn_decode_step.  The state is read once
   and written once per call. */
typedef struct gdn_decode_tokens_args {
  uint32_t struct_size;          /* = sizeof(gdn_decode_tokens_args) */
  int32_t num_seqs;              /* N >= 0 */
  int32_t tokens_per_seq;        /* T >= 0; N*T must fit in int32 */
  int32_t h_k, h_v, d_k, d_v;
  int32_t io_dtype, out_dtype, gate_mode;
  const void* q;                 /* [N*T, h_k, d_k] */
  const void* k;                 /* [N*T, h_k, d_k] */
  const void* v;                 /* [N*T, h_v, d_v] */
  const float* g;                /* [N*T, h_v] */
  const float* beta;             /* [N*T, h_v] */
  const float* A_log;            /* [h_v] (RAW mode) */
  const float* dt_bias;          /* [h_v] (RAW mode) */
  float* state;                  /* [N, h_v, d_v, d_k] fp32, in place: on
                                    return, the state after token T-1
                                    (unchanged when T = 0) */
  float* state_snapshots;        /* [N, T, h_v, d_v, d_k] fp32: the state
                                    after each token, or NULL (not written);
                                    must not overlap any other buffer */
  const void* z;                 /* [N*T, h_v, d_v] io dtype, or NULL */
  const float* norm_weight;      /* [d_v], required when z != NULL */
  float eps;
  void* out;                     /* o [N*T, h_v, d_v] or gated
                                    [N*T, h_v * d_v] */
} gdn_decode_tokens_args;

/* The layer's prologue in front of the recurrence ("A Node-by-Node
   White-Box Walkthrough of a Quantized Hybrid Gated DeltaNet Language Model",
   Principais Contribuicoes: short convolutions precede the gates and the
   recurrent scan; the width is not given and is a parameter here).
   x holds, per token, the channels of q (h_k*d_k), k (h_k*d_k) and v
   (h_v*d_v), in that order (C channels).  Per channel c, within each packed
   sequence:
     y[t, c] = SiLU(bias[c] + sum_{j<W} weight[c, j] * xe[t - (W-1) + j, c]),
   xe being the sequence's input extended on the left by its initial
   convolution state (oldest first) or zeros; then q and k are normalized
   per (token, head): y / sqrt(sum_head y^2 + eps).  The final convolution
   state of a sequence is its last W-1 extended inputs (a later call, e.g. a
   decode step with one token per sequence, continues from it). */
typedef struct gdn_prologue_args {
  uint32_t struct_size;          /* = sizeof(gdn_prologue_args) */
  int32_t num_seqs;              /* N >= 0 (1 when cu_seqlens is NULL) */
  int64_t total_tokens;          /* T >= 0, <= INT32_MAX */
  const int32_t* cu_seqlens;     /* device [N+1] offsets, or NULL: one
                                    sequence of T tokens */
  const int32_t* cu_seqlens_host;/* optional host copy, checked when given */
  int32_t h_k, h_v, d_k, d_v;
  int32_t width;                 /* W in 1..8 */
  int32_t io_dtype, out_dtype;
  const void* x;                 /* [T, C] io dtype */
  const float* weight;           /* [C, W] fp32 */
  const float* bias;             /* [C] fp32, or NULL (no bias) */
  const float* initial_conv_state; /* [N, C, W-1] fp32, or NULL (zeros) */
  float* final_conv_state;       /* [N, C, W-1] fp32, or NULL; must not
                                    overlap initial_conv_state */
  float eps;                     /* L2-normalization epsilon (inside the root) */
  void* q;                       /* [T, h_k, d_k] out dtype */
  void* k;                       /* [T, h_k, d_k] out dtype */
  void* v;                       /* [T, h_v, d_v] out dtype */
} gdn_prologue_args;

/* Standalone gated RMSNorm over rows of d values:
   out[r, i] = x[r, i] * (mean_i x[r, :]^2 + eps)^(-1/2) * w[i] * SiLU(z[r, i]). */
typedef struct gdn_rmsnorm_args {
  uint32_t struct_size;          /* = sizeof(gdn_rmsnorm_args) */
  int32_t d;                     /* row length */
  int64_t rows;                  /* number of rows >= 0 */
  int32_t x_dtype, z_dtype, out_dtype;
  const void* x;                 /* [rows, d] */
  const void* z;                 /* [rows, d] */
  const float* weight;           /* [d] fp32 */
  float eps;
  void* out;                     /* [rows, d]; may equal x when the dtypes
                                    match (in place), otherwise disjoint */
} gdn_rmsnorm_args;

/* Weight formats of the output projection. */
enum {
  GDN_WEIGHT_BF16 = 0,   /* dense bf16 [N, K] */
  GDN_WEIGHT_Q4K = 1,    /* Q4_K blocks (see gdn_out_proj_args) */
  GDN_WEIGHT_FP8 = 2,    /* E4M3 codes [N, K] + fp32 row scales [N];
                            activations quantized per token (W8A8) */
  GDN_WEIGHT_MXFP4 = 3   /* E2M1 codes [N, K/2] (even k in the low nibble)
                            + E8M0 block scales [N, K/32]; activations
                            quantized the same way (W4A4) */
};

/* Output projection after the gated tail ("Red Lite dev15d -- DeltaNet gated
   tail + Q4_K output projection", Pinned graph semantics step 6: the
   flattened 4096-value gated output times ssm_out gives the 2048-value
   hidden vector; "Q4_K implementation": the weight may stay in its packed
   144-byte blocks, decoded on the GPU).
     out[m, n] = sum_k x[m, k] * W[n, k]
   W is [out_features, in_features]:
     GDN_WEIGHT_BF16: dense bf16, row-major;
     GDN_WEIGHT_Q4K:  each row is in_features / 256 consecutive Q4_K blocks
       of 144 bytes (fp16 d, fp16 dmin, 12 bytes of six-bit sub-block scales
       and mins, 128 bytes of four-bit quants; value = d * scale * q -
       dmin * min per 32-value sub-block, GGUF bit order), rows back to back.
   Activations that bf16 does not hold exactly (fp32 x, decoded Q4_K values)
   enter the matrix cores as bf16 parts; accumulation is fp32.
   Low-precision weights ("Why Gated DeltaNet Survives 4-Bit Quantization",
   Abstract: 4-bit weights and activations under block scaling on every
   linear layer, the recurrence kept in high precision) use the OCP formats
   this GPU's matrix cores take natively:
     GDN_WEIGHT_FP8:   out = sx[m] * sw[n] * sum_k e4m3(xq[m, k]) e4m3(W[n, k]),
       sx[m] = 2^e the smallest power of two (e >= -126) with
       max_k |x[m, k]| / 2^e <= 448, xq = x / 2^e rounded to nearest even;
     GDN_WEIGHT_MXFP4: out = sum_k e2m1(xq[m, k]) 2^(xs[m, k/32] - 127)
       e2m1(W[n, k]) 2^(ws[n, k/32] - 127), per 32-value block of x the E8M0
       scale xs = 127 + floor(log2 max|x|) - 2 (0..254; 127 for zeros) and
       xq = x / 2^(xs - 127) rounded to nearest even, saturating at 6.
   The activations are quantized by the call (gdn_quantize_act), in the
   workspace. */
typedef struct gdn_out_proj_args {
  uint32_t struct_size;          /* = sizeof(gdn_out_proj_args) */
  int32_t in_features;           /* K: multiple of 64 (BF16), 256 (Q4K,
                                    MXFP4) or 128 (FP8) */
  int64_t rows;                  /* M >= 0 tokens, <= INT32_MAX */
  int32_t out_features;          /* N >= 1, multiple of 4 */
  int32_t x_dtype, out_dtype;    /* GDN_F32 or GDN_BF16 each */
  int32_t weight_format;         /* GDN_WEIGHT_* */
  const void* x;                 /* [M, K] x dtype */
  const void* weight;            /* see above */
  const void* weight_scale;      /* FP8: fp32 [N]; MXFP4: uint8 [N, K/32];
                                    NULL for BF16 and Q4K */
  void* out;                     /* [M, N] out dtype; must not overlap x,
                                    weight or weight_scale */
} gdn_out_proj_args;

/* Activation quantization of the FP8 / MXFP4 projections (formats as in
   gdn_out_proj_args), on its own: x [rows, cols] ->
     GDN_WEIGHT_FP8:   codes uint8 [rows, cols], scales fp32 [rows] (2^e);
     GDN_WEIGHT_MXFP4: codes uint8 [rows, cols/2], scales uint8 [rows, cols/32]. */
typedef struct gdn_quant_args {
  uint32_t struct_size;          /* = sizeof(gdn_quant_args) */
  int32_t format;                /* GDN_WEIGHT_FP8 or GDN_WEIGHT_MXFP4 */
  int64_t rows;                  /* >= 0, <= INT32_MAX */
  int32_t cols;                  /* multiple of 8 (FP8) or 32 (MXFP4) */
  int32_t x_dtype;               /* GDN_F32 or GDN_BF16 */
  const void* x;
  void* codes;                   /* must not overlap x */
  void* scales;                  /* must not overlap x or codes */
} gdn_quant_args;

/* Library identity. */
uint32_t gdn_abi_version(void);
const char* gdn_status_str(int status);

/* Host-only argument checks (no HIP call; usable without a GPU).  They
   return exactly the code the matching entry point would return before
   launching anything. */
int gdn_validate_prefill(const gdn_prefill_args* args);
int gdn_validate_decode(const gdn_decode_args* args);
int gdn_validate_decode_tokens(const gdn_decode_tokens_args* args);
int gdn_validate_prologue(const gdn_prologue_args* args);
int gdn_validate_rmsnorm(const gdn_rmsnorm_args* args);
int gdn_validate_out_proj(const gdn_out_proj_args* args);
int gdn_validate_quantize_act(const gdn_quant_args* args);

/* Bytes of device workspace gdn_chunk_prefill needs for these arguments
   (0 when none).  Host-only. */
int gdn_prefill_workspace_size(const gdn_prefill_args* args, size_t* bytes);

/* Chunked prefill (WY/UT form of the delta rule, chunk length args->chunk;
   in exact arithmetic the result equals the token-by-token rule above).
   workspace: device buffer of at least gdn_prefill_workspace_size() bytes,
   16-byte aligned and disjoint from every other buffer of the call
   (GDN_E_ALIAS otherwise), or NULL when that size is 0.  The bf16 kernel
   orders its work so that the longest sequences start first; with z set
   its workgroups (the 8 slices of a head's state) exchange the tail's sums
   of squares while they run, so it is launched cooperatively with no more
   workgroups than the device holds at once (GDN_E_HIP if that launch
   fails).  Supported:
     io_dtype BF16, d_k = d_v = 128, chunk 64      -> bf16 MFMA kernel;
     io_dtype F32 or BF16, d_k = d_v in {16, 32, 64, 128},
       chunk in {16, 32, 64}                       -> fp32 VALU kernel.
   Other combinations return GDN_E_UNSUPPORTED. */
int gdn_chunk_prefill(const gdn_prefill_args* args, void* workspace,
                      size_t ws_bytes, void* stream);

/* Bytes of the static scratch behind gdn_chunk_prefill_noalloc. */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* gdn_chunk_prefill without a workspace argument, for callers that cannot
   allocate device memory or pass one (code under HIP graph capture, tight
   serving loops, harnesses that forbid allocation).  The call allocates
   nothing: its workspace is a static array of GDN_NOALLOC_SCRATCH_BYTES
   that the library holds on each GPU it runs on until the process ends.
   Arguments, results and errors are those of gdn_chunk_prefill, plus
   GDN_E_SCRATCH (nothing launched) when gdn_prefill_workspace_size()
   exceeds GDN_NOALLOC_SCRATCH_BYTES: e.g. one 4096-token sequence with 8
   value heads and no tail fits, 32768 tokens with 32 heads do not.
   Every call on one GPU uses that GPU's same array, and the array keeps
   the last call's contents (nothing in it has to start at zero): calls
   that may overlap in time on one GPU (different streams, or host threads
   without ordering) race and give wrong results; calls ordered on one
   stream are safe.  The first call on each GPU looks up that GPU's array
   address (host-side, once; GDN_E_HIP if the lookup fails). */
int gdn_chunk_prefill_noalloc(const gdn_prefill_args* args, void* stream);

/* One decode step, state updated in place (memory-bound single pass over
   the state).  Supported: d_k, d_v in {16, 32, 64, 128}. */
int gdn_decode_step(const gdn_decode_args* args, void* stream);

/* T decode tokens per sequence (see gdn_decode_tokens_args), with the
   optional per-token state snapshots.  Supported: d_k, d_v in
   {16, 32, 64, 128}.  Errors as gdn_decode_step; nothing is launched when
   N*T = 0. */
int gdn_decode_tokens(const gdn_decode_tokens_args* args, void* stream);

/* Convolution prologue (see gdn_prologue_args).  Supported: d_k, d_v in
   {16, 32, 64, 128}, W in 1..8.  Memory-bound single pass over x. */
int gdn_conv_prologue(const gdn_prologue_args* args, void* stream);

/* Standalone gated RMSNorm.  Supported: d in {16, 32, 64, 128, 256}. */
int gdn_gated_rmsnorm(const gdn_rmsnorm_args* args, void* stream);

/* Bytes of device workspace gdn_out_proj needs for these arguments: the
   quantized activations for FP8 / MXFP4, plus fp32 split-K partial sums for
   9 to 4096 rows; for a Q4K weight against BF16 activations beyond 4096
   rows, the weight decoded into two bf16 parts (out_features x in_features
   x 4 bytes).  0 for BF16 / Q4K up to 8 rows and for BF16 beyond 4096.
   Host-only. */
int gdn_out_proj_workspace_size(const gdn_out_proj_args* args, size_t* bytes);

/* Output projection (see gdn_out_proj_args).  BF16 / Q4K weights, up to 8
   rows: one fp32 matrix-vector pass over the weight; more rows: bf16
   matrix-core tiles (beyond 4096 rows with BF16 activations, a Q4K weight
   is first decoded into the workspace as two bf16 parts).  FP8 / MXFP4
   weights: the activations are quantized into the workspace, then fp8 /
   fp4 matrix-core tiles run.  From 9 to 4096 rows K is split over
   workgroups (fp32 partial sums in the workspace, summed in a fixed order,
   so results are deterministic).
   workspace: device buffer of at least gdn_out_proj_workspace_size() bytes,
   16-byte aligned, disjoint from x, weight, weight_scale and out, or NULL
   when that size is 0.  Nothing is launched when rows = 0. */
int gdn_out_proj(const gdn_out_proj_args* args, void* workspace,
                 size_t ws_bytes, void* stream);

/* Activation quantization (see gdn_quant_args).  Memory-bound, one read of
   x (two reads of each row for FP8 rows longer than 4096 values).  Nothing
   is launched when rows = 0. */
int gdn_quantize_act(const gdn_quant_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
