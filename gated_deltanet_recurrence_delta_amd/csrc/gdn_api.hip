// gdn_api.hip -- the C ABI of libgdn.so (declared in include/gdn.h): host-side
// argument validation, kernel selection and launch.  Validation touches no
// HIP API, so it is callable (and tested) on a machine without a GPU.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/gdn.h"
#include "gdn_internal.h"
#include "gdn_proj.h"

namespace {

using gdn::Bf16Plan;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int32_t d) { return d == GDN_F32 || d == GDN_BF16; }

size_t dtype_bytes(int32_t d) { return d == GDN_BF16 ? 2 : 4; }

bool is_pow2_head(int32_t d) {
  return d == 16 || d == 32 || d == 64 || d == 128;
}

// [lo, hi) byte ranges of the buffers one call reads or writes.
struct Range {
  const char* lo;
  const char* hi;
};

Range range(const void* p, size_t bytes) {
  const char* c = static_cast<const char*>(p);
  return Range{c, c + bytes};
}

bool overlap(Range a, Range b) {
  if (!a.lo || !b.lo || a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

enum class PrefillKernel { kNone, kF32, kBf16Mfma };

PrefillKernel select_prefill(const gdn_prefill_args* a) {
  if (gdn::kHaveBf16Mfma && a->io_dtype == GDN_BF16 && a->d_k == 128 &&
      a->d_v == 128 && a->chunk == 64)
    return PrefillKernel::kBf16Mfma;
  if (a->d_k == a->d_v && is_pow2_head(a->d_k) &&
      (a->chunk == 16 || a->chunk == 32 || a->chunk == 64))
    return PrefillKernel::kF32;
  return PrefillKernel::kNone;
}

int validate_prefill(const gdn_prefill_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_prefill_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->io_dtype) || !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  if (a->gate_mode != GDN_GATES_RAW && a->gate_mode != GDN_GATES_DIRECT)
    return GDN_E_DTYPE;
  if (a->num_seqs < 1 || a->total_tokens < 0 ||
      a->total_tokens > (int64_t)INT32_MAX)
    return GDN_E_SHAPE;
  if (a->h_k < 1 || a->h_v < 1 || a->h_v % a->h_k != 0) return GDN_E_SHAPE;
  if (a->d_k < 1 || a->d_v < 1 || a->chunk < 1) return GDN_E_SHAPE;
  if (!a->cu_seqlens && a->total_tokens % a->num_seqs != 0) return GDN_E_SHAPE;
  if (a->cu_seqlens_host) {
    const int32_t* cu = a->cu_seqlens_host;
    if (cu[0] != 0 || (int64_t)cu[a->num_seqs] != a->total_tokens)
      return GDN_E_SHAPE;
    for (int i = 0; i < a->num_seqs; ++i)
      if (cu[i + 1] < cu[i]) return GDN_E_SHAPE;
    // Without device offsets the kernels split T evenly; a host copy that
    // describes other boundaries would be silently ignored.
    if (!a->cu_seqlens) {
      const int64_t len = a->total_tokens / a->num_seqs;
      for (int i = 0; i <= a->num_seqs; ++i)
        if ((int64_t)cu[i] != (int64_t)i * len) return GDN_E_SHAPE;
    }
  }
  if (!(a->eps >= 0.0f)) return GDN_E_SHAPE;
  const bool has_tokens = a->total_tokens > 0;
  if (has_tokens && (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out))
    return GDN_E_NULL;
  if (has_tokens && a->gate_mode == GDN_GATES_RAW && (!a->A_log || !a->dt_bias))
    return GDN_E_NULL;
  if (a->z && !a->norm_weight) return GDN_E_NULL;
  if (select_prefill(a) == PrefillKernel::kNone) return GDN_E_UNSUPPORTED;
  const void* ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->A_log, a->dt_bias,
                        a->initial_state, a->final_state, a->z,
                        a->norm_weight, a->out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_E_ALIGN;
  // Aliasing: out and final_state must not overlap the inputs or each other;
  // final_state may be exactly initial_state (in-place carry).
  const int64_t T = a->total_tokens;
  const size_t io = dtype_bytes(a->io_dtype);
  const size_t st_bytes =
      (size_t)a->num_seqs * a->h_v * a->d_v * a->d_k * sizeof(float);
  const Range rq = range(a->q, (size_t)T * a->h_k * a->d_k * io);
  const Range rk = range(a->k, (size_t)T * a->h_k * a->d_k * io);
  const Range rv = range(a->v, (size_t)T * a->h_v * a->d_v * io);
  const Range rz = range(a->z, a->z ? (size_t)T * a->h_v * a->d_v * io : 0);
  const Range rg = range(a->g, (size_t)T * a->h_v * sizeof(float));
  const Range rb = range(a->beta, (size_t)T * a->h_v * sizeof(float));
  const Range rw = range(a->norm_weight, a->z ? a->d_v * sizeof(float) : 0);
  const Range rs0 = range(a->initial_state, st_bytes);
  const Range rsF = range(a->final_state, st_bytes);
  const Range ro = range(a->out, (size_t)T * a->h_v * a->d_v *
                                     dtype_bytes(a->out_dtype));
  const Range inputs[] = {rq, rk, rv, rz, rg, rb, rw, rs0};
  for (const Range& r : inputs) {
    if (overlap(ro, r)) return GDN_E_ALIAS;
    if (&r != &inputs[7] && overlap(rsF, r)) return GDN_E_ALIAS;
  }
  if (overlap(ro, rsF)) return GDN_E_ALIAS;
  if (a->final_state && a->initial_state &&
      a->final_state != a->initial_state && overlap(rsF, rs0))
    return GDN_E_ALIAS;
  return GDN_OK;
}

// Whether the workspace overlaps any buffer of the call (inputs, out,
// initial or final state); the prefill writes its records there.
bool prefill_ws_overlaps(const gdn_prefill_args* a, Range ws) {
  const int64_t T = a->total_tokens;
  const size_t io = dtype_bytes(a->io_dtype);
  const size_t st_bytes =
      (size_t)a->num_seqs * a->h_v * a->d_v * a->d_k * sizeof(float);
  const Range rs[] = {
      range(a->q, (size_t)T * a->h_k * a->d_k * io),
      range(a->k, (size_t)T * a->h_k * a->d_k * io),
      range(a->v, (size_t)T * a->h_v * a->d_v * io),
      range(a->z, a->z ? (size_t)T * a->h_v * a->d_v * io : 0),
      range(a->g, (size_t)T * a->h_v * sizeof(float)),
      range(a->beta, (size_t)T * a->h_v * sizeof(float)),
      range(a->A_log, a->A_log ? (size_t)a->h_v * sizeof(float) : 0),
      range(a->dt_bias, a->dt_bias ? (size_t)a->h_v * sizeof(float) : 0),
      range(a->norm_weight, a->z ? a->d_v * sizeof(float) : 0),
      range(a->cu_seqlens, a->cu_seqlens ? (size_t)(a->num_seqs + 1) * 4 : 0),
      range(a->initial_state, st_bytes),
      range(a->final_state, st_bytes),
      range(a->out, (size_t)T * a->h_v * a->d_v * dtype_bytes(a->out_dtype))};
  for (const Range& r : rs)
    if (overlap(ws, r)) return true;
  return false;
}

size_t prefill_ws_bytes(const gdn_prefill_args* a) {
  if (select_prefill(a) == PrefillKernel::kBf16Mfma)
    return gdn::plan_prefill_bf16(a->total_tokens, a->num_seqs, a->h_k,
                                  a->h_v, a->d_v, a->z != nullptr)
        .ws_bytes;
  return 0;
}

int validate_decode(const gdn_decode_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_decode_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->io_dtype) || !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  if (a->gate_mode != GDN_GATES_RAW && a->gate_mode != GDN_GATES_DIRECT)
    return GDN_E_DTYPE;
  if (a->num_seqs < 0 || a->h_k < 1 || a->h_v < 1 || a->h_v % a->h_k != 0 ||
      a->d_k < 1 || a->d_v < 1)
    return GDN_E_SHAPE;
  if (!(a->eps >= 0.0f)) return GDN_E_SHAPE;
  if (a->num_seqs > 0) {
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->state || !a->out)
      return GDN_E_NULL;
    if (a->gate_mode == GDN_GATES_RAW && (!a->A_log || !a->dt_bias))
      return GDN_E_NULL;
  }
  if (a->z && !a->norm_weight) return GDN_E_NULL;
  if (!is_pow2_head(a->d_k) || !is_pow2_head(a->d_v)) return GDN_E_UNSUPPORTED;
  const void* ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->A_log,
                        a->dt_bias, a->state, a->z, a->norm_weight, a->out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_E_ALIGN;
  const int64_t N = a->num_seqs;
  const size_t io = dtype_bytes(a->io_dtype);
  const Range rs = range(a->state, (size_t)N * a->h_v * a->d_v * a->d_k * 4);
  const Range ro =
      range(a->out, (size_t)N * a->h_v * a->d_v * dtype_bytes(a->out_dtype));
  const Range ins[] = {
      range(a->q, (size_t)N * a->h_k * a->d_k * io),
      range(a->k, (size_t)N * a->h_k * a->d_k * io),
      range(a->v, (size_t)N * a->h_v * a->d_v * io),
      range(a->z, a->z ? (size_t)N * a->h_v * a->d_v * io : 0),
      range(a->g, (size_t)N * a->h_v * 4),
      range(a->beta, (size_t)N * a->h_v * 4),
      range(a->norm_weight, a->z ? (size_t)a->d_v * 4 : 0)};
  for (const Range& r : ins)
    if (overlap(ro, r) || overlap(rs, r)) return GDN_E_ALIAS;
  if (overlap(ro, rs)) return GDN_E_ALIAS;
  return GDN_OK;
}

int validate_decode_tokens(const gdn_decode_tokens_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_decode_tokens_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->io_dtype) || !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  if (a->gate_mode != GDN_GATES_RAW && a->gate_mode != GDN_GATES_DIRECT)
    return GDN_E_DTYPE;
  if (a->num_seqs < 0 || a->tokens_per_seq < 0 || a->h_k < 1 || a->h_v < 1 ||
      a->h_v % a->h_k != 0 || a->d_k < 1 || a->d_v < 1)
    return GDN_E_SHAPE;
  if ((int64_t)a->num_seqs * a->tokens_per_seq > INT32_MAX) return GDN_E_SHAPE;
  if (!(a->eps >= 0.0f)) return GDN_E_SHAPE;
  const int64_t NT = (int64_t)a->num_seqs * a->tokens_per_seq;
  if (a->num_seqs > 0 && !a->state) return GDN_E_NULL;
  if (NT > 0) {
    if (!a->q || !a->k || !a->v || !a->g || !a->beta || !a->out)
      return GDN_E_NULL;
    if (a->gate_mode == GDN_GATES_RAW && (!a->A_log || !a->dt_bias))
      return GDN_E_NULL;
  }
  if (a->z && !a->norm_weight) return GDN_E_NULL;
  if (!is_pow2_head(a->d_k) || !is_pow2_head(a->d_v)) return GDN_E_UNSUPPORTED;
  const void* ptrs[] = {a->q, a->k, a->v, a->g, a->beta, a->A_log, a->dt_bias,
                        a->state, a->state_snapshots, a->z, a->norm_weight,
                        a->out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_E_ALIGN;
  const int64_t N = a->num_seqs;
  const size_t io = dtype_bytes(a->io_dtype);
  const size_t head_state = (size_t)a->h_v * a->d_v * a->d_k * 4;
  const Range rs = range(a->state, (size_t)N * head_state);
  const Range rn = range(a->state_snapshots,
                         a->state_snapshots ? (size_t)NT * head_state : 0);
  const Range ro =
      range(a->out, (size_t)NT * a->h_v * a->d_v * dtype_bytes(a->out_dtype));
  const Range ins[] = {
      range(a->q, (size_t)NT * a->h_k * a->d_k * io),
      range(a->k, (size_t)NT * a->h_k * a->d_k * io),
      range(a->v, (size_t)NT * a->h_v * a->d_v * io),
      range(a->z, a->z ? (size_t)NT * a->h_v * a->d_v * io : 0),
      range(a->g, (size_t)NT * a->h_v * 4),
      range(a->beta, (size_t)NT * a->h_v * 4),
      range(a->norm_weight, a->z ? (size_t)a->d_v * 4 : 0)};
  for (const Range& r : ins)
    if (overlap(ro, r) || overlap(rs, r) || overlap(rn, r)) return GDN_E_ALIAS;
  if (overlap(ro, rs) || overlap(rn, rs) || overlap(rn, ro)) return GDN_E_ALIAS;
  return GDN_OK;
}

int validate_prologue(const gdn_prologue_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_prologue_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->io_dtype) || !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  if (a->num_seqs < 0 || a->total_tokens < 0 ||
      a->total_tokens > (int64_t)INT32_MAX)
    return GDN_E_SHAPE;
  if (!a->cu_seqlens && a->num_seqs > 1) return GDN_E_SHAPE;
  if (a->num_seqs == 0 && a->total_tokens != 0) return GDN_E_SHAPE;
  if (a->h_k < 1 || a->h_v < 1 || a->h_v % a->h_k != 0 || a->d_k < 1 ||
      a->d_v < 1 || a->width < 1)
    return GDN_E_SHAPE;
  if (a->cu_seqlens_host) {
    const int32_t* cu = a->cu_seqlens_host;
    if (cu[0] != 0 || (int64_t)cu[a->num_seqs] != a->total_tokens)
      return GDN_E_SHAPE;
    for (int i = 0; i < a->num_seqs; ++i)
      if (cu[i + 1] < cu[i]) return GDN_E_SHAPE;
  }
  if (!(a->eps >= 0.0f)) return GDN_E_SHAPE;
  const int64_t T = a->total_tokens;
  if (T > 0 && (!a->x || !a->weight || !a->q || !a->k || !a->v))
    return GDN_E_NULL;
  if (!is_pow2_head(a->d_k) || !is_pow2_head(a->d_v) || a->width > 8)
    return GDN_E_UNSUPPORTED;
  const void* ptrs[] = {a->x, a->weight, a->bias, a->initial_conv_state,
                        a->final_conv_state, a->q, a->k, a->v};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_E_ALIGN;
  const int64_t C = 2 * (int64_t)a->h_k * a->d_k + (int64_t)a->h_v * a->d_v;
  const size_t io = dtype_bytes(a->io_dtype), od = dtype_bytes(a->out_dtype);
  const size_t st = (size_t)a->num_seqs * C * (a->width - 1) * sizeof(float);
  const Range rs0 = range(a->initial_conv_state, a->initial_conv_state ? st : 0);
  const Range rsf = range(a->final_conv_state, a->final_conv_state ? st : 0);
  const Range ins[] = {
      range(a->x, (size_t)T * C * io),
      range(a->weight, (size_t)C * a->width * sizeof(float)),
      range(a->bias, a->bias ? (size_t)C * sizeof(float) : 0), rs0};
  const Range outs[] = {
      range(a->q, (size_t)T * a->h_k * a->d_k * od),
      range(a->k, (size_t)T * a->h_k * a->d_k * od),
      range(a->v, (size_t)T * a->h_v * a->d_v * od), rsf};
  for (const Range& o : outs) {
    for (const Range& i : ins)
      if (overlap(o, i)) return GDN_E_ALIAS;
    for (const Range& o2 : outs)
      if (&o != &o2 && overlap(o, o2)) return GDN_E_ALIAS;
  }
  return GDN_OK;
}

int validate_rmsnorm(const gdn_rmsnorm_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_rmsnorm_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->x_dtype) || !valid_dtype(a->z_dtype) ||
      !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  if (a->rows < 0 || a->d < 1) return GDN_E_SHAPE;
  if (!(a->eps >= 0.0f)) return GDN_E_SHAPE;
  if (a->rows > 0 && (!a->x || !a->z || !a->weight || !a->out))
    return GDN_E_NULL;
  if (!(is_pow2_head(a->d) || a->d == 256)) return GDN_E_UNSUPPORTED;
  const void* ptrs[] = {a->x, a->z, a->weight, a->out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return GDN_E_ALIGN;
  const size_t n = (size_t)a->rows * a->d;
  const Range rx = range(a->x, n * dtype_bytes(a->x_dtype));
  const Range rz = range(a->z, n * dtype_bytes(a->z_dtype));
  const Range rw = range(a->weight, (size_t)a->d * 4);
  const Range ro = range(a->out, n * dtype_bytes(a->out_dtype));
  const bool in_place = a->out == a->x && a->out_dtype == a->x_dtype;
  if (!in_place && overlap(ro, rx)) return GDN_E_ALIAS;
  if (overlap(ro, rz) || overlap(ro, rw)) return GDN_E_ALIAS;
  return GDN_OK;
}

// Bytes of each projection operand (the weight and its scales).
size_t proj_weight_bytes(const gdn_out_proj_args* a) {
  const size_t K = (size_t)a->in_features, N = (size_t)a->out_features;
  switch (a->weight_format) {
    case GDN_WEIGHT_Q4K: return N * (K / 256) * 144;
    case GDN_WEIGHT_FP8: return N * K;
    case GDN_WEIGHT_MXFP4: return N * K / 2;
    default: return N * K * 2;
  }
}

size_t proj_scale_bytes(const gdn_out_proj_args* a) {
  const size_t K = (size_t)a->in_features, N = (size_t)a->out_features;
  if (a->weight_format == GDN_WEIGHT_FP8) return N * sizeof(float);
  if (a->weight_format == GDN_WEIGHT_MXFP4) return N * K / 32;
  return 0;
}

int validate_out_proj(const gdn_out_proj_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_out_proj_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->x_dtype) || !valid_dtype(a->out_dtype))
    return GDN_E_DTYPE;
  const int32_t f = a->weight_format;
  if (f != GDN_WEIGHT_BF16 && f != GDN_WEIGHT_Q4K && f != GDN_WEIGHT_FP8 &&
      f != GDN_WEIGHT_MXFP4)
    return GDN_E_DTYPE;
  if (a->rows < 0 || a->rows > (int64_t)INT32_MAX || a->in_features < 1 ||
      a->out_features < 1)
    return GDN_E_SHAPE;
  const int kmul = f == GDN_WEIGHT_BF16 ? 64 : (f == GDN_WEIGHT_FP8 ? 128 : 256);
  if (a->in_features % kmul != 0 || a->out_features % 4 != 0)
    return GDN_E_SHAPE;
  if (a->rows == 0) return GDN_OK;
  const bool scaled = f == GDN_WEIGHT_FP8 || f == GDN_WEIGHT_MXFP4;
  if (!a->x || !a->weight || !a->out || (scaled && !a->weight_scale))
    return GDN_E_NULL;
  if (!aligned16(a->x) || !aligned16(a->weight) || !aligned16(a->out) ||
      (scaled && !aligned16(a->weight_scale)))
    return GDN_E_ALIGN;
  const size_t M = (size_t)a->rows, K = (size_t)a->in_features,
               N = (size_t)a->out_features;
  const Range rx = range(a->x, M * K * dtype_bytes(a->x_dtype));
  const Range rw = range(a->weight, proj_weight_bytes(a));
  const Range rs = range(scaled ? a->weight_scale : nullptr,
                         proj_scale_bytes(a));
  const Range ro = range(a->out, M * N * dtype_bytes(a->out_dtype));
  if (overlap(ro, rx) || overlap(ro, rw) || overlap(ro, rs)) return GDN_E_ALIAS;
  return GDN_OK;
}

int validate_quant(const gdn_quant_args* a) {
  if (!a) return GDN_E_NULL;
  if (a->struct_size != sizeof(gdn_quant_args)) return GDN_E_STRUCT;
  if (!valid_dtype(a->x_dtype)) return GDN_E_DTYPE;
  if (a->format != GDN_WEIGHT_FP8 && a->format != GDN_WEIGHT_MXFP4)
    return GDN_E_DTYPE;
  const bool fp8 = a->format == GDN_WEIGHT_FP8;
  if (a->rows < 0 || a->rows > (int64_t)INT32_MAX || a->cols < 1 ||
      a->cols % (fp8 ? 8 : 32) != 0)
    return GDN_E_SHAPE;
  if (a->rows == 0) return GDN_OK;
  if (!a->x || !a->codes || !a->scales) return GDN_E_NULL;
  // x rows of 8 (FP8) or 32 values are 16-byte multiples in either dtype;
  // FP8 code rows are 8-byte multiples, MXFP4 ones 16.
  if (!aligned16(a->x) || !aligned16(a->codes) || !aligned16(a->scales))
    return GDN_E_ALIGN;
  const size_t M = (size_t)a->rows, K = (size_t)a->cols;
  const Range rx = range(a->x, M * K * dtype_bytes(a->x_dtype));
  const Range rc = range(a->codes, fp8 ? M * K : M * K / 2);
  const Range rs = range(a->scales, fp8 ? M * sizeof(float) : M * K / 32);
  if (overlap(rc, rx) || overlap(rs, rx) || overlap(rs, rc)) return GDN_E_ALIAS;
  return GDN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_E_HIP; }

}  // namespace

extern "C" {

uint32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_E_NULL: return "a required pointer is NULL";
    case GDN_E_SHAPE: return "invalid or inconsistent sizes";
    case GDN_E_DTYPE: return "unknown dtype or gate mode";
    case GDN_E_UNSUPPORTED: return "combination not supported by this library";
    case GDN_E_ALIGN: return "pointer not 16-byte aligned";
    case GDN_E_WORKSPACE: return "workspace missing or too small";
    case GDN_E_HIP: return "HIP runtime error";
    case GDN_E_STRUCT: return "argument struct size mismatch";
    case GDN_E_ALIAS: return "output overlaps an input";
    case GDN_E_SCRATCH:
      return "request needs more workspace than the library's static scratch";
  }
  return "unknown status";
}

int gdn_validate_prefill(const gdn_prefill_args* a) {
  return validate_prefill(a);
}

int gdn_validate_decode(const gdn_decode_args* a) { return validate_decode(a); }

int gdn_validate_decode_tokens(const gdn_decode_tokens_args* a) {
  return validate_decode_tokens(a);
}

int gdn_validate_prologue(const gdn_prologue_args* a) {
  return validate_prologue(a);
}

int gdn_validate_rmsnorm(const gdn_rmsnorm_args* a) {
  return validate_rmsnorm(a);
}

int gdn_validate_out_proj(const gdn_out_proj_args* a) {
  return validate_out_proj(a);
}

int gdn_validate_quantize_act(const gdn_quant_args* a) {
  return validate_quant(a);
}

int gdn_out_proj_workspace_size(const gdn_out_proj_args* a, size_t* bytes) {
  if (!bytes) return GDN_E_NULL;
  const int st = validate_out_proj(a);
  if (st != GDN_OK) return st;
  *bytes = a->rows == 0
               ? 0
               : gdn::plan_out_proj(a->rows, a->in_features, a->out_features,
                                    a->weight_format, a->x_dtype == GDN_F32)
                     .ws_bytes;
  return GDN_OK;
}

int gdn_out_proj(const gdn_out_proj_args* a, void* workspace,
                 size_t ws_bytes, void* stream) {
  const int st = validate_out_proj(a);
  if (st != GDN_OK) return st;
  if (a->rows == 0) return GDN_OK;
  const gdn::ProjPlan plan =
      gdn::plan_out_proj(a->rows, a->in_features, a->out_features,
                         a->weight_format, a->x_dtype == GDN_F32);
  if (plan.ws_bytes > 0 &&
      (!workspace || ws_bytes < plan.ws_bytes || !aligned16(workspace)))
    return GDN_E_WORKSPACE;
  if (plan.ws_bytes > 0) {
    const Range rw = range(workspace, plan.ws_bytes);
    const size_t M = (size_t)a->rows, K = (size_t)a->in_features,
                 N = (size_t)a->out_features;
    if (overlap(rw, range(a->x, M * K * dtype_bytes(a->x_dtype))) ||
        overlap(rw, range(a->weight, proj_weight_bytes(a))) ||
        overlap(rw, range(a->weight_scale, proj_scale_bytes(a))) ||
        overlap(rw, range(a->out, M * N * dtype_bytes(a->out_dtype))))
      return GDN_E_ALIAS;
  }
  char* ws = static_cast<char*>(workspace);
  gdn::ProjParams p{};
  p.splits = plan.splits;
  p.ws = plan.splits > 1 ? reinterpret_cast<float*>(ws + plan.slab_off) : nullptr;
  const bool lp = a->weight_format == GDN_WEIGHT_FP8 ||
                  a->weight_format == GDN_WEIGHT_MXFP4;
  p.xq = lp ? reinterpret_cast<uint8_t*>(ws + plan.xq_off) : nullptr;
  p.xs = lp ? static_cast<void*>(ws + plan.xs_off) : nullptr;
  p.wd = plan.kernel == gdn::ProjKernel::kGemm && a->weight_format == GDN_WEIGHT_Q4K
             ? reinterpret_cast<uint16_t*>(ws + plan.wd_off)
             : nullptr;
  p.x = a->x;
  p.w = a->weight;
  p.wscale = a->weight_scale;
  p.out = a->out;
  p.M = a->rows;
  p.K = a->in_features;
  p.N = a->out_features;
  p.x_bf16 = a->x_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.wfmt = a->weight_format;
  return hip_status(gdn::launch_out_proj(p, static_cast<hipStream_t>(stream)));
}

int gdn_quantize_act(const gdn_quant_args* a, void* stream) {
  const int st = validate_quant(a);
  if (st != GDN_OK) return st;
  gdn::QuantParams q{};
  q.x = a->x;
  q.codes = static_cast<uint8_t*>(a->codes);
  q.scales = a->scales;
  q.M = a->rows;
  q.K = a->cols;
  q.x_bf16 = a->x_dtype == GDN_BF16;
  q.fmt = a->format;
  return hip_status(gdn::launch_quantize(q, static_cast<hipStream_t>(stream)));
}

int gdn_prefill_workspace_size(const gdn_prefill_args* a, size_t* bytes) {
  if (!bytes) return GDN_E_NULL;
  const int st = validate_prefill(a);
  if (st != GDN_OK) return st;
  *bytes = prefill_ws_bytes(a);
  return GDN_OK;
}

namespace {

// Launches a validated prefill with `workspace` (at least
// prefill_ws_bytes(a) bytes, or NULL when that is 0).
int run_prefill(const gdn_prefill_args* a, void* workspace, void* stream) {
  gdn::PrefillParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.s0 = a->initial_state;
  p.sF = a->final_state;
  p.z = a->z;
  p.w = a->norm_weight;
  p.out = a->out;
  p.cu = a->cu_seqlens;
  p.ws = static_cast<float*>(workspace);
  p.T = a->total_tokens;
  p.N = a->num_seqs;
  p.seq_len = a->cu_seqlens ? 0 : (int32_t)(a->total_tokens / a->num_seqs);
  p.h_k = a->h_k;
  p.h_v = a->h_v;
  p.group = a->h_v / a->h_k;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.chunk = a->chunk;
  p.io_bf16 = a->io_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.direct = a->gate_mode == GDN_GATES_DIRECT;
  p.tail = a->z != nullptr;
  p.eps = a->eps;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (select_prefill(a) == PrefillKernel::kBf16Mfma) {
    p.slices =
        gdn::plan_prefill_bf16(p.T, p.N, p.h_k, p.h_v, p.d_v, p.tail).slices;
    return hip_status(gdn::launch_prefill_bf16(p, s));
  }
  return hip_status(gdn::launch_prefill_f32(p, s));
}

}  // namespace

int gdn_chunk_prefill(const gdn_prefill_args* a, void* workspace,
                      size_t ws_bytes, void* stream) {
  const int st = validate_prefill(a);
  if (st != GDN_OK) return st;
  const size_t need = prefill_ws_bytes(a);
  if (need > 0 && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return GDN_E_WORKSPACE;
  if (need > 0 && prefill_ws_overlaps(a, range(workspace, need)))
    return GDN_E_ALIAS;
  return run_prefill(a, workspace, stream);
}

// ------------------------------------------------ no-allocation prefill --
// The workspace of gdn_chunk_prefill_noalloc: one array per GPU, created
// when the code object is loaded on that GPU and held until the process
// ends.  In host code `scratch` is only a handle for the symbol lookup: its
// device address on each GPU comes from hipGetSymbolAddress, made once per
// device with that device current, and only that address is handed to
// kernels.
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GDN_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return GDN_E_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return GDN_OK;
}

}  // namespace

int gdn_chunk_prefill_noalloc(const gdn_prefill_args* a, void* stream) {
  const int st = validate_prefill(a);
  if (st != GDN_OK) return st;
  const size_t need = prefill_ws_bytes(a);
  if (need > GDN_NOALLOC_SCRATCH_BYTES) return GDN_E_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int sa = scratch_address(&ws);
    if (sa != GDN_OK) return sa;
  }
  return run_prefill(a, ws, stream);
}

int gdn_decode_step(const gdn_decode_args* a, void* stream) {
  const int st = validate_decode(a);
  if (st != GDN_OK) return st;
  gdn::DecodeParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.state = a->state;
  p.snaps = nullptr;
  p.z = a->z;
  p.w = a->norm_weight;
  p.out = a->out;
  p.N = a->num_seqs;
  p.T = 1;
  p.h_k = a->h_k;
  p.h_v = a->h_v;
  p.group = a->h_v / a->h_k;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.io_bf16 = a->io_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.direct = a->gate_mode == GDN_GATES_DIRECT;
  p.tail = a->z != nullptr;
  p.eps = a->eps;
  return hip_status(gdn::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int gdn_decode_tokens(const gdn_decode_tokens_args* a, void* stream) {
  const int st = validate_decode_tokens(a);
  if (st != GDN_OK) return st;
  gdn::DecodeParams p{};
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.g = a->g;
  p.beta = a->beta;
  p.A_log = a->A_log;
  p.dt_bias = a->dt_bias;
  p.state = a->state;
  p.snaps = a->state_snapshots;
  p.z = a->z;
  p.w = a->norm_weight;
  p.out = a->out;
  p.N = a->num_seqs;
  p.T = a->tokens_per_seq;
  p.h_k = a->h_k;
  p.h_v = a->h_v;
  p.group = a->h_v / a->h_k;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.io_bf16 = a->io_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.direct = a->gate_mode == GDN_GATES_DIRECT;
  p.tail = a->z != nullptr;
  p.eps = a->eps;
  return hip_status(gdn::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int gdn_conv_prologue(const gdn_prologue_args* a, void* stream) {
  const int st = validate_prologue(a);
  if (st != GDN_OK) return st;
  gdn::PrologueParams p{};
  p.x = a->x;
  p.w = a->weight;
  p.bias = a->bias;
  p.cu = a->cu_seqlens;
  p.s0 = a->initial_conv_state;
  p.sF = a->final_conv_state;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.T = a->total_tokens;
  p.C = 2 * (int64_t)a->h_k * a->d_k + (int64_t)a->h_v * a->d_v;
  p.N = a->num_seqs;
  p.h_k = a->h_k;
  p.h_v = a->h_v;
  p.d_k = a->d_k;
  p.d_v = a->d_v;
  p.W = a->width;
  p.io_bf16 = a->io_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.eps = a->eps;
  if (p.N == 0) return GDN_OK;
  return hip_status(gdn::launch_prologue(p, static_cast<hipStream_t>(stream)));
}

int gdn_gated_rmsnorm(const gdn_rmsnorm_args* a, void* stream) {
  const int st = validate_rmsnorm(a);
  if (st != GDN_OK) return st;
  gdn::RmsParams p{};
  p.x = a->x;
  p.z = a->z;
  p.w = a->weight;
  p.out = a->out;
  p.rows = a->rows;
  p.d = a->d;
  p.x_bf16 = a->x_dtype == GDN_BF16;
  p.z_bf16 = a->z_dtype == GDN_BF16;
  p.out_bf16 = a->out_dtype == GDN_BF16;
  p.eps = a->eps;
  return hip_status(gdn::launch_rmsnorm(p, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
