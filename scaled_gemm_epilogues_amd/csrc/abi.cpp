// C ABI of libsge: argument validation (host only, before any HIP call) and dispatch.
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <string>

#include "../../include/sge.h"
#include "launch.h"

namespace {

thread_local std::string g_msg;

sge_status fail(sge_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

sge_status ok() {
  g_msg.clear();
  return SGE_OK;
}

sge_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SGE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_size(int fmt) { return fmt == SGE_FMT_BF16 ? 2 : 1; }

// Byte range [lo, hi) touched by a row-major matrix.
struct Range {
  uintptr_t lo, hi;
};
Range range_of(const void* p, int64_t rows, int64_t cols, int64_t ld, int es) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  if (rows <= 0 || cols <= 0) return {b, b};
  return {b, b + (uintptr_t)(((rows - 1) * ld + cols) * es)};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

Range operand_range(const sge_operand& o) {
  const int64_t rows = o.inner_contiguous ? o.outer : o.inner;
  const int64_t cols = o.inner_contiguous ? o.inner : o.outer;
  return range_of(o.data, rows, cols, o.ld, elem_size(o.format));
}

// Checks one GEMM operand in the order NULL, shape, format, alignment.
sge_status check_operand(const sge_operand* o, const char* name) {
  if (!o) return fail(SGE_ERR_NULL, "%s: operand descriptor is NULL", name);
  if (o->outer < 0 || o->inner < 0) return fail(SGE_ERR_SHAPE, "%s: negative size", name);
  const bool empty = o->outer == 0 || o->inner == 0;
  if (!empty && !o->data) return fail(SGE_ERR_NULL, "%s: data is NULL", name);
  if (o->format == SGE_FMT_E4M3 && !o->scale_inv) return fail(SGE_ERR_NULL, "%s: scale_inv is NULL", name);
  if (o->format == SGE_FMT_MXFP8 && !empty && !o->mx_scale)
    return fail(SGE_ERR_NULL, "%s: mx_scale is NULL", name);
  const int64_t min_ld = o->inner_contiguous ? o->inner : o->outer;
  if (o->ld < min_ld || o->ld <= 0) return fail(SGE_ERR_SHAPE, "%s: ld %lld < %lld", name, (long long)o->ld,
                                                (long long)min_ld);
  switch (o->format) {
    case SGE_FMT_BF16:
      if (o->inner_contiguous && o->inner % 8)
        return fail(SGE_ERR_SHAPE, "%s: bf16 contraction dim %lld not a multiple of 8", name, (long long)o->inner);
      if (!o->inner_contiguous && o->outer % 8)
        return fail(SGE_ERR_SHAPE, "%s: bf16 transposed operand needs outer %% 8 == 0 (got %lld)", name,
                    (long long)o->outer);
      break;
    case SGE_FMT_E4M3:
      if (!o->inner_contiguous) return fail(SGE_ERR_FORMAT, "%s: E4M3 operands must be inner-contiguous", name);
      if (o->inner % 16)
        return fail(SGE_ERR_SHAPE, "%s: E4M3 contraction dim %lld not a multiple of 16", name, (long long)o->inner);
      break;
    case SGE_FMT_MXFP8:
      if (!o->inner_contiguous) return fail(SGE_ERR_FORMAT, "%s: MXFP8 operands must be inner-contiguous", name);
      if (o->inner % 32)
        return fail(SGE_ERR_SHAPE, "%s: MXFP8 contraction dim %lld not a multiple of 32", name, (long long)o->inner);
      if (o->mx_ld < o->inner / 32) return fail(SGE_ERR_SHAPE, "%s: mx_ld too small", name);
      break;
    default:
      return fail(SGE_ERR_FORMAT, "%s: unknown format %d", name, o->format);
  }
  if (!aligned16(o->data) || (o->ld * elem_size(o->format)) % 16)
    return fail(SGE_ERR_ALIGN, "%s: data or ld not 16-byte aligned", name);
  return SGE_OK;
}

// The GEMM kernels address each operand, output and scale array through buffer resources with
// 32-bit byte offsets, counted from a tile's first row (from a k-tile's first contraction row for
// the transposed bf16 operands); a resource spans at most kMaxSpan bytes. A row stride is
// accepted when 256 rows of it (plus the tile's contraction bytes) fit, and the arrays a kernel
// addresses from one base (MXFP8 scale arrays, a gated weight's two halves) must fit whole.
// Larger shapes are refused (SGE_ERR_SHAPE) rather than read as zeros.
constexpr int64_t kMaxSpan = 0x7FFFFF00;
constexpr int64_t kMaxRowBytes = (kMaxSpan - 4096) / 257;

sge_status check_strides(const char* what, std::initializer_list<int64_t> row_bytes) {
  for (int64_t b : row_bytes)
    if (b > kMaxRowBytes)
      return fail(SGE_ERR_SHAPE, "%s: a row stride of %lld bytes exceeds the kernels' 32-bit tile addressing (%lld)",
                  what, (long long)b, (long long)kMaxRowBytes);
  return SGE_OK;
}

sge_status check_span(const char* what, int64_t bytes) {
  if (bytes > kMaxSpan)
    return fail(SGE_ERR_SHAPE, "%s: an array of %lld bytes exceeds the kernels' 32-bit addressing (%lld)", what,
                (long long)bytes, (long long)kMaxSpan);
  return SGE_OK;
}

// A token-blocked output written by a grouped epilogue: the layout, and ld as the token-blocked
// quantizer takes it (every group's range fits below ld). Addressed with 64-bit pointers.
sge_status check_colT(const char* what, int64_t T, int32_t G, const int64_t* layout, int64_t ld, const void* q,
                      const void* sc) {
  if (!layout) return fail(SGE_ERR_NULL, "%s: a token-blocked output needs the group layout", what);
  if (G > 4096) return fail(SGE_ERR_ARG, "%s: G=%d outside [1, 4096]", what, G);
  if (ld % SGE_MX_TOKEN_ALIGN || ld < sge_mx_token_capacity(T, G))
    return fail(SGE_ERR_SHAPE, "%s: ld_t=%lld must be a multiple of %d and >= sge_mx_token_capacity(T, G)=%lld", what,
                (long long)ld, SGE_MX_TOKEN_ALIGN, (long long)sge_mx_token_capacity(T, G));
  if (!aligned16(q) || !aligned16(sc)) return fail(SGE_ERR_ALIGN, "%s: pointers must be 16-byte aligned", what);
  return SGE_OK;
}

sge::GemmParams gemm_params(const sge_operand& a, const sge_operand& b, void* c, int64_t ldc, float alpha,
                            int accumulate) {
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(a.data);
  p.lda = a.ld;
  p.b = static_cast<const uint8_t*>(b.data);
  p.ldb = b.ld;
  p.M = a.outer;
  p.N = b.outer;
  p.K = a.inner;
  p.a_sinv = a.scale_inv;
  p.b_sinv = b.scale_inv;
  p.a_mx = a.mx_scale;
  p.a_mx_ld = a.mx_ld;
  p.b_mx = b.mx_scale;
  p.b_mx_ld = b.mx_ld;
  p.mx_aligned = (a.inner % 128 == 0) && (a.mx_ld % 4 == 0) && (b.mx_ld % 4 == 0) &&
                 ((reinterpret_cast<uintptr_t>(a.mx_scale) & 3u) == 0) &&
                 ((reinterpret_cast<uintptr_t>(b.mx_scale) & 3u) == 0);
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(c);
  p.ldc = ldc;
  p.accumulate = accumulate;
  return p;
}

// Validates the pair (a, b) of one GEMM producing bf16 C [a.outer, b.outer].
sge_status check_gemm(const sge_operand* a, const sge_operand* b, const void* c, int64_t ldc, const char* what) {
  sge_status s = check_operand(a, "A");
  if (s != SGE_OK) return s;
  if ((s = check_operand(b, "B")) != SGE_OK) return s;
  if (a->inner != b->inner)
    return fail(SGE_ERR_SHAPE, "%s: contraction dims differ (%lld vs %lld)", what, (long long)a->inner,
                (long long)b->inner);
  if (a->format != b->format) return fail(SGE_ERR_FORMAT, "%s: operand formats differ", what);
  if (a->outer > 0 && b->outer > 0 && !c) return fail(SGE_ERR_NULL, "%s: output is NULL", what);
  if (b->outer % 8) return fail(SGE_ERR_SHAPE, "%s: output columns %lld not a multiple of 8", what,
                                (long long)b->outer);
  if (ldc < b->outer) return fail(SGE_ERR_SHAPE, "%s: output ld too small", what);
  if ((s = check_strides(what, {a->ld * elem_size(a->format), b->ld * elem_size(b->format), ldc * 2})) != SGE_OK)
    return s;
  if (a->format == SGE_FMT_MXFP8 &&
      ((s = check_span(what, a->outer * a->mx_ld)) != SGE_OK || (s = check_span(what, b->outer * b->mx_ld)) != SGE_OK))
    return s;
  if (c && (!aligned16(c) || (ldc * 2) % 16)) return fail(SGE_ERR_ALIGN, "%s: output not 16-byte aligned", what);
  const int64_t tiles = ((a->outer + 255) / 256) * ((b->outer + 255) / 256);
  if (tiles > 0x7FFFFFFF) return fail(SGE_ERR_SHAPE, "%s: too many tiles", what);
  return SGE_OK;
}

}  // namespace

// Epilogues the grouped calls take. Gated ones split the pre-activation into two halves.
bool fwd_epilogue_ok(int32_t e) {
  return e == SGE_EPI_NONE || e == SGE_EPI_SCALED_SWIGLU || e == SGE_EPI_SCALED_SRELU ||
         e == SGE_EPI_SCALED_CLAMPED_SWIGLU;
}
bool bwd_epilogue_ok(int32_t e) {
  return e == SGE_EPI_NONE || e == SGE_EPI_DSCALED_SWIGLU || e == SGE_EPI_DSCALED_SRELU ||
         e == SGE_EPI_DSCALED_CLAMPED_SWIGLU;
}
bool gated_fwd(int32_t e) { return e == SGE_EPI_SCALED_SWIGLU || e == SGE_EPI_SCALED_CLAMPED_SWIGLU; }
bool gated_bwd(int32_t e) { return e == SGE_EPI_DSCALED_SWIGLU || e == SGE_EPI_DSCALED_CLAMPED_SWIGLU; }
bool clamped(int32_t e) { return e == SGE_EPI_SCALED_CLAMPED_SWIGLU || e == SGE_EPI_DSCALED_CLAMPED_SWIGLU; }

// The clamped SwiGLU needs its parameters: limit > 0 and finite, alpha finite.
sge_status check_act(int32_t e, const sge_act_params* act, const char* what) {
  if (!clamped(e)) return SGE_OK;
  if (!act) return fail(SGE_ERR_NULL, "%s: the clamped SwiGLU needs act (limit, alpha)", what);
  if (!(act->limit > 0.0f) || !std::isfinite(act->limit) || !std::isfinite(act->alpha))
    return fail(SGE_ERR_ARG, "%s: clamped SwiGLU limit must be finite and > 0, alpha finite", what);
  return SGE_OK;
}

void set_act(sge::GemmParams& p, int32_t e, const sge_act_params* act) {
  if (clamped(e)) {
    p.act_limit = act->limit;
    p.act_alpha = act->alpha;
  }
}

extern "C" {

int sge_abi_version(void) { return SGE_ABI_VERSION; }

const char* sge_status_string(sge_status s) {
  switch (s) {
    case SGE_OK: return "SGE_OK";
    case SGE_ERR_NULL: return "SGE_ERR_NULL";
    case SGE_ERR_SHAPE: return "SGE_ERR_SHAPE";
    case SGE_ERR_FORMAT: return "SGE_ERR_FORMAT";
    case SGE_ERR_ALIGN: return "SGE_ERR_ALIGN";
    case SGE_ERR_ALIAS: return "SGE_ERR_ALIAS";
    case SGE_ERR_WORKSPACE: return "SGE_ERR_WORKSPACE";
    case SGE_ERR_ARG: return "SGE_ERR_ARG";
    case SGE_ERR_HIP: return "SGE_ERR_HIP";
  }
  return "unknown sge_status";
}

const char* sge_last_error_message(void) { return g_msg.c_str(); }

sge_status sge_linear_scale_add_fwd(const sge_operand* x, const sge_operand* w, void* residual, int64_t ld_res,
                                    float alpha, int32_t accumulate, hipStream_t stream) {
  sge_status s = check_gemm(x, w, residual, ld_res, "linear_scale_add_fwd");
  if (s != SGE_OK) return s;
  const Range out = range_of(residual, x->outer, w->outer, ld_res, 2);
  if (overlap(out, operand_range(*x)) || overlap(out, operand_range(*w)))
    return fail(SGE_ERR_ALIAS, "linear_scale_add_fwd: residual overlaps x or w");
  if (x->outer == 0 || w->outer == 0) return ok();
  if (alpha == 0.0f) {
    if (accumulate) return ok();   // the residual is the result, bit for bit
    return hip_status(sge::launch_fill_bf16_zero(static_cast<uint16_t*>(residual), x->outer, w->outer, ld_res,
                                                 stream),
                      "fill");
  }
  if (x->inner == 0) {
    if (accumulate) return ok();
    return hip_status(sge::launch_fill_bf16_zero(static_cast<uint16_t*>(residual), x->outer, w->outer, ld_res,
                                                 stream),
                      "fill");
  }
  sge::GemmParams p = gemm_params(*x, *w, residual, ld_res, alpha, accumulate ? 1 : 0);
  return hip_status(sge::launch_gemm(p, x->format, x->inner_contiguous != 0, w->inner_contiguous != 0, stream),
                    "gemm launch");
}

sge_status sge_linear_scale_bwd(const sge_operand* dg_a, const sge_operand* dg_b, const sge_operand* wg_a,
                                const sge_operand* wg_b, void* dgrad, int64_t ld_dgrad, void* wgrad,
                                int64_t ld_wgrad, float dgrad_alpha, float wgrad_alpha, hipStream_t stream) {
  sge_status s;
  if (dgrad) {
    if ((s = check_gemm(dg_a, dg_b, dgrad, ld_dgrad, "dgrad")) != SGE_OK) return s;
  }
  if (wgrad) {
    if ((s = check_gemm(wg_a, wg_b, wgrad, ld_wgrad, "wgrad")) != SGE_OK) return s;
  }
  if (dgrad && wgrad) {
    if (dg_a->outer != wg_b->inner || dg_b->outer != wg_b->outer || wg_a->outer != dg_a->inner)
      return fail(SGE_ERR_SHAPE, "backward: dgrad [M,N]x[K,N] and wgrad [N,M]x[K,M] shapes disagree");
  }
  if (dgrad) {
    const Range out = range_of(dgrad, dg_a->outer, dg_b->outer, ld_dgrad, 2);
    if (overlap(out, operand_range(*dg_a)) || overlap(out, operand_range(*dg_b)) ||
        (wgrad && (overlap(out, operand_range(*wg_a)) || overlap(out, operand_range(*wg_b)))))
      return fail(SGE_ERR_ALIAS, "dgrad overlaps an input");
  }
  if (wgrad) {
    const Range out = range_of(wgrad, wg_a->outer, wg_b->outer, ld_wgrad, 2);
    if (overlap(out, operand_range(*wg_a)) || overlap(out, operand_range(*wg_b)) ||
        (dgrad && (overlap(out, operand_range(*dg_a)) || overlap(out, operand_range(*dg_b)))))
      return fail(SGE_ERR_ALIAS, "wgrad overlaps an input");
    if (dgrad && overlap(out, range_of(dgrad, dg_a->outer, dg_b->outer, ld_dgrad, 2)))
      return fail(SGE_ERR_ALIAS, "wgrad overlaps dgrad");
  }
  if (dgrad && dg_a->outer > 0 && dg_b->outer > 0) {
    hipError_t e;
    if (dgrad_alpha == 0.0f || dg_a->inner == 0) {
      e = sge::launch_fill_bf16_zero(static_cast<uint16_t*>(dgrad), dg_a->outer, dg_b->outer, ld_dgrad, stream);
    } else {
      sge::GemmParams p = gemm_params(*dg_a, *dg_b, dgrad, ld_dgrad, dgrad_alpha, 0);
      e = sge::launch_gemm(p, dg_a->format, dg_a->inner_contiguous != 0, dg_b->inner_contiguous != 0, stream);
    }
    if (e != hipSuccess) return hip_status(e, "dgrad launch");
  }
  if (wgrad && wg_a->outer > 0 && wg_b->outer > 0) {
    hipError_t e;
    if (wgrad_alpha == 0.0f || wg_a->inner == 0) {
      e = sge::launch_fill_bf16_zero(static_cast<uint16_t*>(wgrad), wg_a->outer, wg_b->outer, ld_wgrad, stream);
    } else {
      sge::GemmParams p = gemm_params(*wg_a, *wg_b, wgrad, ld_wgrad, wgrad_alpha, 0);
      e = sge::launch_gemm(p, wg_a->format, wg_a->inner_contiguous != 0, wg_b->inner_contiguous != 0, stream);
    }
    if (e != hipSuccess) return hip_status(e, "wgrad launch");
  }
  return ok();
}

size_t sge_quantize_fp8_amax_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return 0;
  return (size_t)sge::amax_partial_blocks(rows * cols) * sizeof(uint32_t);
}

// Validation (NULL, shape, alignment, alias), then the two launches; the partials go to
// `workspace`, or, with workspace == NULL, to this GPU's scratch array.
static sge_status quantize_fp8_amax_impl(const char* what, const void* src, int64_t rows, int64_t cols, uint8_t* q,
                                         uint8_t* q_t, float* amax, float* scale, float* scale_inv, void* workspace,
                                         size_t workspace_bytes, bool scratch, hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "%s: negative size", what);
  if ((rows * cols > 0 && !src) || !amax || !scale || !scale_inv || (!scratch && !workspace))
    return fail(SGE_ERR_NULL, "%s: NULL pointer", what);
  if (rows % 16 || cols % 16) return fail(SGE_ERR_SHAPE, "%s: rows and cols must be multiples of 16", what);
  if (sge_status st = check_strides(what, {cols * 2})) return st;   // 128-row tiles, 32-bit offsets
  if (!aligned16(src) || (q && !aligned16(q)) || (q_t && !aligned16(q_t)))
    return fail(SGE_ERR_ALIGN, "%s: pointers must be 16-byte aligned", what);
  const Range in = range_of(src, rows, cols, cols, 2);
  if ((q && overlap(in, range_of(q, rows, cols, cols, 1))) || (q_t && overlap(in, range_of(q_t, cols, rows, rows, 1))))
    return fail(SGE_ERR_ALIAS, "%s: output overlaps the input", what);
  const size_t need = sge_quantize_fp8_amax_workspace_size(rows, cols);
  if (scratch) {
    uint32_t* ws = nullptr;
    hipError_t e = sge::amax_scratch(&ws, &workspace_bytes);
    if (e != hipSuccess) return hip_status(e, "scratch array address");
    if (workspace_bytes < need)
      return fail(SGE_ERR_WORKSPACE, "%s: %zu bytes of amax partials exceed the %zu-byte scratch array", what, need,
                  workspace_bytes);
    workspace = ws;
  } else if (workspace_bytes < need) {
    return fail(SGE_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", what, workspace_bytes, need);
  }
  const int nb = sge::amax_partial_blocks(rows * cols);
  hipError_t e = sge::launch_amax_partial(static_cast<const uint16_t*>(src), rows * cols,
                                          static_cast<uint32_t*>(workspace), nb, stream);
  if (e != hipSuccess) return hip_status(e, "amax launch");
  e = sge::launch_quantize_fp8(static_cast<const uint16_t*>(src), rows, cols, static_cast<const uint32_t*>(workspace),
                               nb, q, q_t, amax, scale, scale_inv, stream);
  return hip_status(e, "quantize launch");
}

sge_status sge_quantize_fp8_amax(const void* src, int64_t rows, int64_t cols, uint8_t* q, uint8_t* q_t, float* amax,
                                 float* scale, float* scale_inv, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return quantize_fp8_amax_impl("quantize_fp8_amax", src, rows, cols, q, q_t, amax, scale, scale_inv, workspace,
                                workspace_bytes, false, stream);
}

sge_status sge_quantize_fp8_amax_noalloc(const void* src, int64_t rows, int64_t cols, uint8_t* q, uint8_t* q_t,
                                         float* amax, float* scale, float* scale_inv, hipStream_t stream) {
  return quantize_fp8_amax_impl("quantize_fp8_amax_noalloc", src, rows, cols, q, q_t, amax, scale, scale_inv,
                                nullptr, 0, true, stream);
}

sge_status sge_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, uint8_t* q_row, uint8_t* s_row,
                              uint8_t* q_colT, uint8_t* s_colT, hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "quantize_mxfp8: negative size");
  const bool want_row = q_row || s_row, want_col = q_colT || s_colT;
  if (!want_row && !want_col) return fail(SGE_ERR_NULL, "quantize_mxfp8: no output requested");
  if ((want_row && (!q_row || !s_row)) || (want_col && (!q_colT || !s_colT)))
    return fail(SGE_ERR_NULL, "quantize_mxfp8: data and scale pointers come in pairs");
  if (rows * cols > 0 && !src) return fail(SGE_ERR_NULL, "quantize_mxfp8: src is NULL");
  if (cols % 32 || (want_col && rows % 32))
    return fail(SGE_ERR_SHAPE, "quantize_mxfp8: cols (and rows, for the columnwise copy) must be multiples of 32");
  if (sge_status st = check_strides("quantize_mxfp8", {cols * 2})) return st;   // 128-row tiles, 32-bit offsets
  if (!aligned16(src) || (q_row && !aligned16(q_row)) || (q_colT && !aligned16(q_colT)))
    return fail(SGE_ERR_ALIGN, "quantize_mxfp8: pointers must be 16-byte aligned");
  const Range in = range_of(src, rows, cols, cols, 2);
  if ((q_row && overlap(in, range_of(q_row, rows, cols, cols, 1))) ||
      (q_colT && overlap(in, range_of(q_colT, cols, rows, rows, 1))))
    return fail(SGE_ERR_ALIAS, "quantize_mxfp8: output overlaps the input");
  if (rows == 0 || cols == 0) return ok();
  return hip_status(sge::launch_quantize_mxfp8(static_cast<const uint16_t*>(src), rows, cols, q_row, s_row, q_colT,
                                               s_colT, stream),
                    "quantize_mxfp8 launch");
}

sge_status sge_splits_to_offsets(const int64_t* splits, int32_t G, const int64_t* multipliers, int32_t n_mult,
                                 int64_t expected_total, int64_t* offsets, int32_t* err_flag, hipStream_t stream) {
  if (!splits || !multipliers || !offsets) return fail(SGE_ERR_NULL, "splits_to_offsets: NULL pointer");
  if (G < 1 || G > 4096) return fail(SGE_ERR_ARG, "splits_to_offsets: G=%d outside [1, 4096]", G);
  if (n_mult < 1 || n_mult > 8) return fail(SGE_ERR_ARG, "splits_to_offsets: n_mult=%d outside [1, 8]", n_mult);
  return hip_status(sge::launch_splits_to_offsets(splits, G, multipliers, n_mult, expected_total, offsets, err_flag,
                                                  stream),
                    "splits_to_offsets launch");
}

sge_status sge_grouped_linear_fwd(const void* x, const void* w, int32_t G, int64_t T, int64_t N, int64_t K,
                                  const int64_t* offsets, float alpha, int32_t epilogue,
                                  const sge_act_params* act_params, const float* probs, void* out, void* preact,
                                  hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd: bad sizes");
  if (!fwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_fwd: epilogue %d not allowed", epilogue);
  if (!x || !w || !offsets || !out) return fail(SGE_ERR_NULL, "grouped_linear_fwd: NULL pointer");
  if (epilogue != SGE_EPI_NONE && !probs) return fail(SGE_ERR_NULL, "grouped_linear_fwd: probs is NULL");
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_fwd")) return st;
  if (K % 8 || N % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd: N and K must be multiples of 8");
  if (gated_fwd(epilogue) && N % 256)
    return fail(SGE_ERR_SHAPE, "grouped_linear_fwd: SwiGLU needs N %% 256 == 0");
  if (sge_status st = check_strides("grouped_linear_fwd", {K * 2, N * 2})) return st;
  if (gated_fwd(epilogue))
    if (sge_status st = check_span("grouped_linear_fwd", (N / 2 + 256) * K * 2)) return st;
  if (!aligned16(x) || !aligned16(w) || !aligned16(out) || (preact && !aligned16(preact)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_fwd: pointers must be 16-byte aligned");
  const int64_t out_cols = gated_fwd(epilogue) ? N / 2 : N;
  const Range ro = range_of(out, T, out_cols, out_cols, 2);
  if (overlap(ro, range_of(x, T, K, K, 2)) || overlap(ro, range_of(w, (int64_t)G * N, K, K, 2)) ||
      (preact && overlap(range_of(preact, T, N, N, 2), ro)))
    return fail(SGE_ERR_ALIAS, "grouped_linear_fwd: outputs overlap inputs");
  if (T == 0 || N == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(x);
  p.lda = K;
  p.b = static_cast<const uint8_t*>(w);
  p.ldb = K;
  p.M = T;
  p.N = N;
  p.K = K;
  p.b_group_stride = N * K;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(out);
  p.ldc = out_cols;
  p.offsets = offsets;
  p.G = G;
  p.T = T;
  p.probs = probs;
  p.aux = static_cast<uint16_t*>(preact);
  p.ld_aux = N;
  p.F = N / 2;
  set_act(p, epilogue, act_params);
  return hip_status(sge::launch_grouped_fwd(p, epilogue, stream), "grouped fwd launch");
}

sge_status sge_grouped_linear_fwd_mxfp8(const void* x_q, const void* x_s, const void* w_q, const void* w_s, int32_t G,
                                        int64_t T, int64_t N, int64_t K, const int64_t* offsets, float alpha,
                                        int32_t epilogue, const sge_act_params* act_params, const float* probs,
                                        void* out, void* preact, void* out_q, void* out_s, const int64_t* layout,
                                        int64_t ld_t, void* out_colT_q, void* out_colT_s, hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_mxfp8: bad sizes");
  if (!fwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_fwd_mxfp8: epilogue %d not allowed", epilogue);
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_fwd_mxfp8")) return st;
  const bool swiglu = gated_fwd(epilogue);
  const bool act = epilogue != SGE_EPI_NONE;                      // a scaled activation in the epilogue
  if (!x_q || !x_s || !w_q || !w_s || !offsets) return fail(SGE_ERR_NULL, "grouped_linear_fwd_mxfp8: NULL pointer");
  if ((out_q == nullptr) != (out_s == nullptr))
    return fail(SGE_ERR_NULL, "grouped_linear_fwd_mxfp8: out_q and out_s go together");
  if (out_q && !act) return fail(SGE_ERR_ARG, "grouped_linear_fwd_mxfp8: a quantized output needs an activation epilogue");
  if ((out_colT_q == nullptr) != (out_colT_s == nullptr))
    return fail(SGE_ERR_NULL, "grouped_linear_fwd_mxfp8: out_colT_q and out_colT_s go together");
  if (out_colT_q && !act)
    return fail(SGE_ERR_ARG, "grouped_linear_fwd_mxfp8: a token-blocked output needs an activation epilogue");
  if (!out && !out_q && !out_colT_q) return fail(SGE_ERR_NULL, "grouped_linear_fwd_mxfp8: no output");
  if (act && !probs) return fail(SGE_ERR_NULL, "grouped_linear_fwd_mxfp8: probs is NULL");
  if (out_q && N % 32) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_mxfp8: an MXFP8 output needs N %% 32 == 0");
  if (K % 128) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_mxfp8: K must be a multiple of 128 (got %lld)", (long long)K);
  if (N % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_mxfp8: N must be a multiple of 8");
  if (swiglu && N % 256) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_mxfp8: SwiGLU needs N %% 256 == 0");
  if (sge_status st = check_strides("grouped_linear_fwd_mxfp8", {K, N * 2})) return st;
  if (swiglu)
    if (sge_status st = check_span("grouped_linear_fwd_mxfp8", (N / 2 + 256) * K)) return st;
  if (sge_status st = check_span("grouped_linear_fwd_mxfp8", T * (K / 32))) return st;
  if (sge_status st = check_span("grouped_linear_fwd_mxfp8", (int64_t)G * N * (K / 32))) return st;
  if (!aligned16(x_q) || !aligned16(x_s) || !aligned16(w_q) || !aligned16(w_s) || (out && !aligned16(out)) ||
      (preact && !aligned16(preact)) || (out_q && !aligned16(out_q)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_fwd_mxfp8: pointers must be 16-byte aligned");
  const int64_t out_cols = swiglu ? N / 2 : N;
  if (out_colT_q)
    if (sge_status st = check_colT("grouped_linear_fwd_mxfp8", T, G, layout, ld_t, out_colT_q, out_colT_s)) return st;
  const Range in[5] = {range_of(x_q, T, K, K, 1), range_of(x_s, T, K / 32, K / 32, 1),
                       range_of(w_q, (int64_t)G * N, K, K, 1), range_of(w_s, (int64_t)G * N, K / 32, K / 32, 1),
                       out_colT_q ? range_of(layout, 2, G + 1, G + 1, 8) : Range{0, 0}};
  const Range outs[6] = {out ? range_of(out, T, out_cols, out_cols, 2) : Range{0, 0},
                         preact ? range_of(preact, T, N, N, 2) : Range{0, 0},
                         out_q ? range_of(out_q, T, out_cols, out_cols, 1) : Range{0, 0},
                         out_s ? range_of(out_s, T, out_cols / 32, out_cols / 32, 1) : Range{0, 0},
                         out_colT_q ? range_of(out_colT_q, out_cols, ld_t, ld_t, 1) : Range{0, 0},
                         out_colT_s ? range_of(out_colT_s, out_cols, ld_t / 32, ld_t / 32, 1) : Range{0, 0}};
  for (const Range& o : outs) {
    for (const Range& i : in)
      if (overlap(o, i)) return fail(SGE_ERR_ALIAS, "grouped_linear_fwd_mxfp8: outputs overlap inputs");
  }
  for (int a = 0; a < 6; ++a)
    for (int b = a + 1; b < 6; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "grouped_linear_fwd_mxfp8: outputs overlap");
  if (T == 0 || N == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(x_q);
  p.lda = K;
  p.b = static_cast<const uint8_t*>(w_q);
  p.ldb = K;
  p.M = T;
  p.N = N;
  p.K = K;
  p.b_group_stride = N * K;
  p.a_mx = static_cast<const uint8_t*>(x_s);
  p.a_mx_ld = K / 32;
  p.b_mx = static_cast<const uint8_t*>(w_s);
  p.b_mx_ld = K / 32;
  p.b_mx_group_stride = N * (K / 32);
  p.mx_aligned = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(out);
  p.ldc = out_cols;
  p.offsets = offsets;
  p.G = G;
  p.T = T;
  p.probs = probs;
  p.aux = static_cast<uint16_t*>(preact);
  p.ld_aux = N;
  p.F = N / 2;
  p.q_out = static_cast<uint8_t*>(out_q);
  p.s_out = static_cast<uint8_t*>(out_s);
  p.ld_q = out_cols;
  p.qt_out = static_cast<uint8_t*>(out_colT_q);
  p.st_out = static_cast<uint8_t*>(out_colT_s);
  p.ld_t = ld_t;
  p.mx_layout = layout;
  set_act(p, epilogue, act_params);
  return hip_status(sge::launch_grouped_fwd_mx(p, epilogue, stream), "grouped fwd mxfp8 launch");
}

size_t sge_grouped_linear_bwd_workspace_size(int64_t T, int64_t K, int32_t G, int32_t epilogue) {
  (void)G;
  if (epilogue == SGE_EPI_NONE || !bwd_epilogue_ok(epilogue) || T <= 0 || K <= 0) return 0;
  const int64_t parts = sge::gemm_dp_parts_per_tile() * ((K + sge::gemm_tile_n() - 1) / sge::gemm_tile_n());
  return (size_t)(parts * T) * sizeof(float);
}

sge_status sge_grouped_linear_bwd(const void* dy, const void* x, const void* w, int32_t G, int64_t T, int64_t N,
                                  int64_t K, const int64_t* offsets, float alpha, int32_t epilogue,
                                  const sge_act_params* act_params, const void* preact, const float* probs,
                                  void* dact, float* dprobs, void* dx, void* dw, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_bwd: bad sizes");
  if (!bwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_bwd: epilogue %d not allowed", epilogue);
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_bwd")) return st;
  const bool swiglu = epilogue != SGE_EPI_NONE;                  // an activation backward in the epilogue
  const int64_t hw = gated_bwd(epilogue) ? 2 * K : K;   // pre-activation / dact width
  if (!dy || !w || !offsets) return fail(SGE_ERR_NULL, "grouped_linear_bwd: NULL pointer");
  if (dw && !x) return fail(SGE_ERR_NULL, "grouped_linear_bwd: x is NULL");
  if (swiglu && (!preact || !probs || !dact || !dprobs))
    return fail(SGE_ERR_NULL, "grouped_linear_bwd: the activation backward needs preact, probs, dact and dprobs");
  if (K % 8 || N % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_bwd: N and K must be multiples of 8");
  if (sge_status st = check_strides("grouped_linear_bwd", {N * 2, K * 2, hw * 2})) return st;
  if (!aligned16(dy) || (x && !aligned16(x)) || !aligned16(w) || (dx && !aligned16(dx)) || (dw && !aligned16(dw)) ||
      (preact && !aligned16(preact)) || (dact && !aligned16(dact)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_bwd: pointers must be 16-byte aligned");
  const Range rdy = range_of(dy, T, N, N, 2), rw = range_of(w, (int64_t)G * N, K, K, 2);
  const Range rx = x ? range_of(x, T, K, K, 2) : Range{0, 0};
  if ((dx && !swiglu && (overlap(range_of(dx, T, K, K, 2), rdy) || overlap(range_of(dx, T, K, K, 2), rw))) ||
      (dw && (overlap(range_of(dw, (int64_t)G * N, K, K, 2), rdy) || overlap(range_of(dw, (int64_t)G * N, K, K, 2), rx))) ||
      (swiglu && (overlap(range_of(dact, T, hw, hw, 2), rdy) ||
                  overlap(range_of(dact, T, hw, hw, 2), range_of(preact, T, hw, hw, 2)))))
    return fail(SGE_ERR_ALIAS, "grouped_linear_bwd: outputs overlap inputs");
  const size_t need = sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SGE_ERR_WORKSPACE, "grouped_linear_bwd: workspace %zu < %zu bytes", workspace_bytes, need);
  if (T == 0) {
    if (dw) return hip_status(sge::launch_fill_bf16_zero(static_cast<uint16_t*>(dw), (int64_t)G * N, K, K, stream), "fill");
    return ok();
  }
  const bool want_dg = swiglu || dx;
  sge::GemmParams pd, pw;
  memset(&pd, 0, sizeof(pd));
  memset(&pw, 0, sizeof(pw));
  if (want_dg) {
    pd.a = static_cast<const uint8_t*>(dy);
    pd.lda = N;
    pd.b = static_cast<const uint8_t*>(w);
    pd.ldb = K;
    pd.M = T;
    pd.N = K;
    pd.K = N;
    pd.b_group_stride = N * K;
    pd.alpha = alpha;
    pd.c = static_cast<uint16_t*>(dx);
    pd.ldc = K;
    pd.offsets = offsets;
    pd.G = G;
    pd.T = T;
    if (swiglu) {
      pd.probs = probs;
      pd.aux = const_cast<uint16_t*>(static_cast<const uint16_t*>(preact));
      pd.ld_aux = hw;
      pd.aux_out = static_cast<uint16_t*>(dact);
      pd.ld_aux_out = hw;
      pd.dp_part = static_cast<float*>(workspace);
      pd.F = K;
    }
    set_act(pd, epilogue, act_params);
  }
  if (dw) {
    pw.a = static_cast<const uint8_t*>(dy);
    pw.lda = N;
    pw.b = static_cast<const uint8_t*>(x);
    pw.ldb = K;
    pw.M = N;
    pw.N = K;
    pw.K = T;
    pw.alpha = alpha;
    pw.c = static_cast<uint16_t*>(dw);
    pw.ldc = K;
    pw.c_group_stride = N * K;
    pw.offsets = offsets;
    pw.G = G;
    pw.T = T;
  }
  // Both GEMMs read only the call's inputs, so they share one launch when both are asked for.
  hipError_t e = hipSuccess;
  if (want_dg && dw) e = sge::launch_grouped_dgrad_wgrad(pd, epilogue, pw, stream);
  else if (want_dg) e = sge::launch_grouped_dgrad(pd, epilogue, stream);
  else if (dw) e = sge::launch_grouped_wgrad(pw, stream);
  if (e != hipSuccess) return hip_status(e, "grouped dgrad / wgrad launch");
  if (swiglu) {
    const int parts = (int)(sge::gemm_dp_parts_per_tile() * ((K + sge::gemm_tile_n() - 1) / sge::gemm_tile_n()));
    e = sge::launch_rowsum_parts(static_cast<const float*>(workspace), parts, offsets, G, T, dprobs, stream);
    if (e != hipSuccess) return hip_status(e, "dprobs reduction launch");
  }
  return ok();
}

int64_t sge_mx_token_capacity(int64_t T, int32_t G) {
  if (T < 0 || G < 1) return -1;
  return (T + SGE_MX_TOKEN_ALIGN - 1) / SGE_MX_TOKEN_ALIGN * SGE_MX_TOKEN_ALIGN + (int64_t)G * SGE_MX_TOKEN_ALIGN;
}

sge_status sge_mx_group_layout(const int64_t* offsets, int32_t G, int64_t T, int64_t* layout, hipStream_t stream) {
  if (!offsets || !layout) return fail(SGE_ERR_NULL, "mx_group_layout: NULL pointer");
  if (G < 1 || G > 4096) return fail(SGE_ERR_ARG, "mx_group_layout: G=%d outside [1, 4096]", G);
  if (T < 0) return fail(SGE_ERR_SHAPE, "mx_group_layout: negative T");
  if (overlap(Range{(uintptr_t)offsets, (uintptr_t)(offsets + G + 1)}, Range{(uintptr_t)layout, (uintptr_t)(layout + 2 * (G + 1))}))
    return fail(SGE_ERR_ALIAS, "mx_group_layout: layout overlaps offsets");
  return hip_status(sge::launch_mx_group_layout(offsets, G, T, SGE_MX_TOKEN_ALIGN, layout, stream),
                    "mx_group_layout launch");
}

sge_status sge_quantize_mxfp8_grouped(const void* src, int64_t T, int64_t cols, int32_t G, const int64_t* layout,
                                      int64_t ld, uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                                      hipStream_t stream) {
  if (T < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "quantize_mxfp8_grouped: negative size");
  if (G < 1 || G > 4096) return fail(SGE_ERR_ARG, "quantize_mxfp8_grouped: G=%d outside [1, 4096]", G);
  if (!layout || !q_colT || !s_colT) return fail(SGE_ERR_NULL, "quantize_mxfp8_grouped: layout, q_colT and s_colT are required");
  if ((q_row == nullptr) != (s_row == nullptr))
    return fail(SGE_ERR_NULL, "quantize_mxfp8_grouped: q_row and s_row go together");
  if (T * cols > 0 && !src) return fail(SGE_ERR_NULL, "quantize_mxfp8_grouped: src is NULL");
  if (cols % 32) return fail(SGE_ERR_SHAPE, "quantize_mxfp8_grouped: cols must be a multiple of 32");
  if (sge_status st = check_strides("quantize_mxfp8_grouped", {cols * 2})) return st;   // 128-row tiles, 32-bit offsets
  if (ld % SGE_MX_TOKEN_ALIGN || ld < sge_mx_token_capacity(T, G))
    return fail(SGE_ERR_SHAPE, "quantize_mxfp8_grouped: ld=%lld must be a multiple of %d and >= sge_mx_token_capacity(T, G)=%lld",
                (long long)ld, SGE_MX_TOKEN_ALIGN, (long long)sge_mx_token_capacity(T, G));
  if ((src && !aligned16(src)) || (q_row && !aligned16(q_row)) || !aligned16(q_colT) || !aligned16(s_colT))
    return fail(SGE_ERR_ALIGN, "quantize_mxfp8_grouped: pointers must be 16-byte aligned");
  const Range in = range_of(src, T, cols, cols, 2);
  const Range outs[4] = {q_row ? range_of(q_row, T, cols, cols, 1) : Range{0, 0},
                         s_row ? range_of(s_row, T, cols / 32, cols / 32, 1) : Range{0, 0},
                         range_of(q_colT, cols, ld, ld, 1), range_of(s_colT, cols, ld / 32, ld / 32, 1)};
  const Range lay{(uintptr_t)layout, (uintptr_t)(layout + 2 * (G + 1))};
  for (int a = 0; a < 4; ++a) {
    if (overlap(outs[a], in) || overlap(outs[a], lay)) return fail(SGE_ERR_ALIAS, "quantize_mxfp8_grouped: output overlaps an input");
    for (int b = a + 1; b < 4; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "quantize_mxfp8_grouped: outputs overlap");
  }
  if (cols == 0) return ok();
  return hip_status(sge::launch_quantize_mxfp8_grouped(static_cast<const uint16_t*>(src), T, cols, G, layout, ld,
                                                       q_row, s_row, q_colT, s_colT, stream),
                    "quantize_mxfp8_grouped launch");
}

sge_status sge_grouped_linear_dgrad_mxfp8(const void* dy_q, const void* dy_s, const void* w_q, const void* w_s,
                                          int32_t G, int64_t T, int64_t N, int64_t K, const int64_t* offsets,
                                          float alpha, int32_t epilogue, const sge_act_params* act_params,
                                          const void* preact, const float* probs,
                                          void* dx, void* dact, float* dprobs, void* dact_q, void* dact_s,
                                          const int64_t* layout, int64_t ld_t, void* dact_colT_q,
                                          void* dact_colT_s, void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_mxfp8: bad sizes");
  if (!bwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_dgrad_mxfp8: epilogue %d not allowed", epilogue);
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_dgrad_mxfp8")) return st;
  const bool swiglu = epilogue != SGE_EPI_NONE;                  // an activation backward in the epilogue
  const int64_t hw = gated_bwd(epilogue) ? 2 * K : K;   // pre-activation / dact width
  if (!dy_q || !dy_s || !w_q || !w_s || !offsets) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: NULL pointer");
  if ((dact_q == nullptr) != (dact_s == nullptr))
    return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: dact_q and dact_s go together");
  if ((dact_colT_q == nullptr) != (dact_colT_s == nullptr))
    return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: dact_colT_q and dact_colT_s go together");
  if (swiglu) {
    if (!preact || !probs || !dprobs) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: an activation backward needs preact, probs and dprobs");
    if (!dact && !dact_q && !dact_colT_q) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: no output");
  } else {
    if (!dx) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_mxfp8: dx is NULL");
    if (dact_q || dact_colT_q)
      return fail(SGE_ERR_ARG, "grouped_linear_dgrad_mxfp8: a quantized output needs an activation backward");
  }
  if (N % 128) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_mxfp8: N must be a multiple of 128 (got %lld)", (long long)N);
  if (K % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_mxfp8: K must be a multiple of 8");
  if (swiglu && K % 32) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_mxfp8: an activation backward needs K %% 32 == 0");
  if (sge_status st = check_strides("grouped_linear_dgrad_mxfp8", {N, (int64_t)G * N, hw * 2})) return st;
  if (sge_status st = check_span("grouped_linear_dgrad_mxfp8", T * (N / 32))) return st;
  if (sge_status st = check_span("grouped_linear_dgrad_mxfp8", K * ((int64_t)G * N / 32))) return st;
  if (!aligned16(dy_q) || !aligned16(dy_s) || !aligned16(w_q) || !aligned16(w_s) || (dx && !aligned16(dx)) ||
      (preact && !aligned16(preact)) || (dact && !aligned16(dact)) || (dact_q && !aligned16(dact_q)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_dgrad_mxfp8: pointers must be 16-byte aligned");
  const int64_t GN = (int64_t)G * N;
  if (dact_colT_q)
    if (sge_status st = check_colT("grouped_linear_dgrad_mxfp8", T, G, layout, ld_t, dact_colT_q, dact_colT_s)) return st;
  const Range in[6] = {range_of(dy_q, T, N, N, 1), range_of(dy_s, T, N / 32, N / 32, 1), range_of(w_q, K, GN, GN, 1),
                       range_of(w_s, K, GN / 32, GN / 32, 1),
                       swiglu ? range_of(preact, T, hw, hw, 2) : Range{0, 0},
                       dact_colT_q ? range_of(layout, 2, G + 1, G + 1, 8) : Range{0, 0}};
  const Range outs[6] = {(dx && !swiglu) ? range_of(dx, T, K, K, 2) : Range{0, 0},
                         (swiglu && dact) ? range_of(dact, T, hw, hw, 2) : Range{0, 0},
                         dact_q ? range_of(dact_q, T, hw, hw, 1) : Range{0, 0},
                         dact_s ? range_of(dact_s, T, hw / 32, hw / 32, 1) : Range{0, 0},
                         dact_colT_q ? range_of(dact_colT_q, hw, ld_t, ld_t, 1) : Range{0, 0},
                         dact_colT_s ? range_of(dact_colT_s, hw, ld_t / 32, ld_t / 32, 1) : Range{0, 0}};
  for (int a = 0; a < 6; ++a) {
    for (const Range& i : in)
      if (overlap(outs[a], i)) return fail(SGE_ERR_ALIAS, "grouped_linear_dgrad_mxfp8: outputs overlap inputs");
    for (int b = a + 1; b < 6; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "grouped_linear_dgrad_mxfp8: outputs overlap");
  }
  const size_t need = sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SGE_ERR_WORKSPACE, "grouped_linear_dgrad_mxfp8: workspace %zu < %zu bytes", workspace_bytes, need);
  if (T == 0 || K == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dy_q);
  p.lda = N;
  p.b = static_cast<const uint8_t*>(w_q);       // W blocked along N: [K][G*N], group g at column g*N
  p.ldb = GN;
  p.M = T;
  p.N = K;
  p.K = N;
  p.b_group_stride = N;
  p.a_mx = static_cast<const uint8_t*>(dy_s);
  p.a_mx_ld = N / 32;
  p.b_mx = static_cast<const uint8_t*>(w_s);
  p.b_mx_ld = GN / 32;
  p.b_mx_group_stride = N / 32;
  p.b_mx_bytes = K * (GN / 32);
  p.mx_aligned = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(swiglu ? nullptr : dx);
  p.ldc = K;
  p.offsets = offsets;
  p.G = G;
  p.T = T;
  if (swiglu) {
    p.probs = probs;
    p.aux = const_cast<uint16_t*>(static_cast<const uint16_t*>(preact));
    p.ld_aux = hw;
    p.aux_out = static_cast<uint16_t*>(dact);
    p.ld_aux_out = hw;
    p.dp_part = static_cast<float*>(workspace);
    p.F = K;
    p.q_out = static_cast<uint8_t*>(dact_q);
    p.s_out = static_cast<uint8_t*>(dact_s);
    p.ld_q = hw;
    p.qt_out = static_cast<uint8_t*>(dact_colT_q);
    p.st_out = static_cast<uint8_t*>(dact_colT_s);
    p.ld_t = ld_t;
    p.mx_layout = layout;
  }
  set_act(p, epilogue, act_params);
  hipError_t e = sge::launch_grouped_dgrad_mx(p, epilogue, stream);
  if (e != hipSuccess) return hip_status(e, "grouped dgrad mxfp8 launch");
  if (swiglu) {
    const int parts = (int)(sge::gemm_dp_parts_per_tile() * ((K + sge::gemm_tile_n() - 1) / sge::gemm_tile_n()));
    e = sge::launch_rowsum_parts(static_cast<const float*>(workspace), parts, offsets, G, T, dprobs, stream);
    if (e != hipSuccess) return hip_status(e, "dprobs reduction launch");
  }
  return ok();
}

sge_status sge_grouped_linear_wgrad_mxfp8(const void* dyT_q, const void* dyT_s, const void* xT_q, const void* xT_s,
                                          int32_t G, int64_t N, int64_t K, const int64_t* layout, int64_t ld,
                                          float alpha, void* dw, hipStream_t stream) {
  if (G < 1 || G > 4096 || N < 0 || K < 0 || ld < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_mxfp8: bad sizes");
  if (!dyT_q || !dyT_s || !xT_q || !xT_s || !layout || !dw) return fail(SGE_ERR_NULL, "grouped_linear_wgrad_mxfp8: NULL pointer");
  if (ld % SGE_MX_TOKEN_ALIGN) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_mxfp8: ld must be a multiple of %d", SGE_MX_TOKEN_ALIGN);
  if (K % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_mxfp8: K must be a multiple of 8");
  if (sge_status st = check_strides("grouped_linear_wgrad_mxfp8", {ld, K * 2})) return st;
  if (sge_status st = check_span("grouped_linear_wgrad_mxfp8", (N > K ? N : K) * (ld / 32))) return st;
  if (!aligned16(dyT_q) || !aligned16(dyT_s) || !aligned16(xT_q) || !aligned16(xT_s) || !aligned16(dw))
    return fail(SGE_ERR_ALIGN, "grouped_linear_wgrad_mxfp8: pointers must be 16-byte aligned");
  const Range rdw = range_of(dw, (int64_t)G * N, K, K, 2);
  const Range in[5] = {range_of(dyT_q, N, ld, ld, 1), range_of(dyT_s, N, ld / 32, ld / 32, 1), range_of(xT_q, K, ld, ld, 1),
                       range_of(xT_s, K, ld / 32, ld / 32, 1),
                       Range{(uintptr_t)layout, (uintptr_t)(layout + 2 * (G + 1))}};
  for (const Range& i : in)
    if (overlap(rdw, i)) return fail(SGE_ERR_ALIAS, "grouped_linear_wgrad_mxfp8: dw overlaps an input");
  if (N == 0 || K == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dyT_q);
  p.lda = ld;
  p.b = static_cast<const uint8_t*>(xT_q);
  p.ldb = ld;
  p.M = N;
  p.N = K;
  p.K = ld;
  p.a_mx = static_cast<const uint8_t*>(dyT_s);
  p.a_mx_ld = ld / 32;
  p.b_mx = static_cast<const uint8_t*>(xT_s);
  p.b_mx_ld = ld / 32;
  p.mx_aligned = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(dw);
  p.ldc = K;
  p.c_group_stride = N * K;
  p.offsets = layout + G + 1;                    // the aligned group starts: each group's contraction range
  p.G = G;
  p.T = ld;
  return hip_status(sge::launch_grouped_wgrad_mx(p, stream), "grouped wgrad mxfp8 launch");
}

size_t sge_quantize_fp8_grouped_workspace_size(int32_t G) {
  return G < 1 ? 0 : (size_t)(((int64_t)G * 4 + 15) / 16 * 16);
}

sge_status sge_quantize_fp8_grouped(const void* src, int64_t rows, int64_t cols, int32_t G, const int64_t* layout,
                                    int64_t ld_t, uint8_t* q, uint8_t* q_t, float* amax, float* scale,
                                    float* scale_inv, const float* amax_in, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (rows < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "quantize_fp8_grouped: negative size");
  if (G < 1 || G > 4096) return fail(SGE_ERR_ARG, "quantize_fp8_grouped: G=%d outside [1, 4096]", G);
  if (!amax || !scale || !scale_inv) return fail(SGE_ERR_NULL, "quantize_fp8_grouped: amax, scale and scale_inv are required");
  if (!q && !q_t) return fail(SGE_ERR_NULL, "quantize_fp8_grouped: no output requested");
  if (rows * cols > 0 && !src) return fail(SGE_ERR_NULL, "quantize_fp8_grouped: src is NULL");
  if (cols % 16) return fail(SGE_ERR_SHAPE, "quantize_fp8_grouped: cols must be a multiple of 16");
  if (sge_status st = check_strides("quantize_fp8_grouped", {cols * 2})) return st;   // 128-row tiles, 32-bit offsets
  if (!layout && (rows % G || (rows / G) % 128))
    return fail(SGE_ERR_SHAPE, "quantize_fp8_grouped: without a layout, rows / G must be a whole multiple of 128");
  int64_t npos = rows;
  if (layout) {
    const int64_t cap = sge_mx_token_capacity(rows, G);
    if (q_t && (ld_t % SGE_MX_TOKEN_ALIGN || ld_t < cap))
      return fail(SGE_ERR_SHAPE, "quantize_fp8_grouped: ld_t=%lld must be a multiple of %d and >= sge_mx_token_capacity=%lld",
                  (long long)ld_t, SGE_MX_TOKEN_ALIGN, (long long)cap);
    npos = q_t ? ld_t : cap;
  } else if (q_t && (ld_t < rows || ld_t % 16)) {
    return fail(SGE_ERR_SHAPE, "quantize_fp8_grouped: ld_t must be >= rows and a multiple of 16");
  }
  if ((src && !aligned16(src)) || (q && !aligned16(q)) || (q_t && !aligned16(q_t)))
    return fail(SGE_ERR_ALIGN, "quantize_fp8_grouped: pointers must be 16-byte aligned");
  const size_t need = amax_in ? 0 : sge_quantize_fp8_grouped_workspace_size(G);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SGE_ERR_WORKSPACE, "quantize_fp8_grouped: workspace %zu < %zu bytes", workspace_bytes, need);
  const Range in[3] = {range_of(src, rows, cols, cols, 2),
                       layout ? Range{(uintptr_t)layout, (uintptr_t)(layout + 2 * (G + 1))} : Range{0, 0},
                       amax_in ? range_of(amax_in, 1, G, G, 4) : Range{0, 0}};
  const Range outs[6] = {q ? range_of(q, rows, cols, cols, 1) : Range{0, 0},
                         q_t ? range_of(q_t, cols, ld_t, ld_t, 1) : Range{0, 0},
                         range_of(amax, 1, G, G, 4), range_of(scale, 1, G, G, 4), range_of(scale_inv, 1, G, G, 4),
                         need ? range_of(workspace, 1, G, G, 4) : Range{0, 0}};
  for (int a = 0; a < 6; ++a) {
    for (const Range& i : in)
      if (overlap(outs[a], i)) return fail(SGE_ERR_ALIAS, "quantize_fp8_grouped: an output overlaps an input");
    for (int b = a + 1; b < 6; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "quantize_fp8_grouped: outputs overlap");
  }
  return hip_status(sge::launch_quantize_fp8_grouped(static_cast<const uint16_t*>(src), rows, cols, G, layout, npos,
                                                     static_cast<float*>(workspace), amax_in, q, q_t, amax, scale,
                                                     scale_inv, stream),
                    "quantize_fp8_grouped launch");
}

sge_status sge_grouped_linear_fwd_fp8(const void* x_q, const float* x_sinv, const void* w_q, const float* w_sinv,
                                      int32_t G, int64_t T, int64_t N, int64_t K, const int64_t* offsets, float alpha,
                                      int32_t epilogue, const sge_act_params* act_params, const float* probs,
                                      void* out, void* preact, float* out_amax, hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_fp8: bad sizes");
  if (!fwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_fwd_fp8: epilogue %d not allowed", epilogue);
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_fwd_fp8")) return st;
  const bool swiglu = gated_fwd(epilogue);
  const bool act = epilogue != SGE_EPI_NONE;
  if (!x_q || !x_sinv || !w_q || !w_sinv || !offsets || !out) return fail(SGE_ERR_NULL, "grouped_linear_fwd_fp8: NULL pointer");
  if (act && !probs) return fail(SGE_ERR_NULL, "grouped_linear_fwd_fp8: probs is NULL");
  if (out_amax && !act) return fail(SGE_ERR_ARG, "grouped_linear_fwd_fp8: out_amax needs an activation epilogue");
  if (K % 16) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_fp8: K must be a multiple of 16");
  if (N % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_fp8: N must be a multiple of 8");
  if (swiglu && N % 256) return fail(SGE_ERR_SHAPE, "grouped_linear_fwd_fp8: SwiGLU needs N %% 256 == 0");
  if (sge_status st = check_strides("grouped_linear_fwd_fp8", {K, N * 2})) return st;
  if (swiglu)
    if (sge_status st = check_span("grouped_linear_fwd_fp8", (N / 2 + 256) * K)) return st;
  if (!aligned16(x_q) || !aligned16(w_q) || !aligned16(out) || (preact && !aligned16(preact)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_fwd_fp8: pointers must be 16-byte aligned");
  const int64_t out_cols = swiglu ? N / 2 : N;
  const Range in[2] = {range_of(x_q, T, K, K, 1), range_of(w_q, (int64_t)G * N, K, K, 1)};
  const Range outs[3] = {range_of(out, T, out_cols, out_cols, 2), preact ? range_of(preact, T, N, N, 2) : Range{0, 0},
                         out_amax ? range_of(out_amax, 1, G, G, 4) : Range{0, 0}};
  for (const Range& o : outs)
    for (const Range& i : in)
      if (overlap(o, i)) return fail(SGE_ERR_ALIAS, "grouped_linear_fwd_fp8: outputs overlap inputs");
  if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2]))
    return fail(SGE_ERR_ALIAS, "grouped_linear_fwd_fp8: outputs overlap");
  if (out_amax) {
    const hipError_t z = sge::launch_fill_f32_zero(out_amax, G, stream);
    if (z != hipSuccess) return hip_status(z, "amax fill");
  }
  if (T == 0 || N == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(x_q);
  p.lda = K;
  p.b = static_cast<const uint8_t*>(w_q);
  p.ldb = K;
  p.M = T;
  p.N = N;
  p.K = K;
  p.b_group_stride = N * K;
  p.a_sinv = x_sinv;
  p.b_sinv = w_sinv;
  p.sinv_per_group = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(out);
  p.ldc = out_cols;
  p.offsets = offsets;
  p.G = G;
  p.T = T;
  p.probs = probs;
  p.aux = static_cast<uint16_t*>(preact);
  p.ld_aux = N;
  p.F = N / 2;
  p.amax_out = out_amax;
  set_act(p, epilogue, act_params);
  return hip_status(sge::launch_grouped_fwd_fp8(p, epilogue, stream), "grouped fwd fp8 launch");
}

sge_status sge_grouped_linear_dgrad_fp8(const void* dy_q, const float* dy_sinv, const void* w_qT, const float* w_sinv,
                                        int32_t G, int64_t T, int64_t N, int64_t K, const int64_t* offsets,
                                        float alpha, int32_t epilogue, const sge_act_params* act_params,
                                        const void* preact, const float* probs,
                                        void* dx, void* dact, float* dprobs, float* dact_amax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (G < 1 || T < 0 || N < 0 || K < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_fp8: bad sizes");
  if (!bwd_epilogue_ok(epilogue))
    return fail(SGE_ERR_ARG, "grouped_linear_dgrad_fp8: epilogue %d not allowed", epilogue);
  if (sge_status st = check_act(epilogue, act_params, "grouped_linear_dgrad_fp8")) return st;
  const bool swiglu = epilogue != SGE_EPI_NONE;                  // an activation backward in the epilogue
  const int64_t hw = gated_bwd(epilogue) ? 2 * K : K;   // pre-activation / dact width
  if (!dy_q || !dy_sinv || !w_qT || !w_sinv || !offsets) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_fp8: NULL pointer");
  if (swiglu && (!preact || !probs || !dact || !dprobs))
    return fail(SGE_ERR_NULL, "grouped_linear_dgrad_fp8: an activation backward needs preact, probs, dact and dprobs");
  if (!swiglu && !dx) return fail(SGE_ERR_NULL, "grouped_linear_dgrad_fp8: dx is NULL");
  if (dact_amax && !swiglu) return fail(SGE_ERR_ARG, "grouped_linear_dgrad_fp8: dact_amax needs an activation backward");
  if (N % 16) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_fp8: N must be a multiple of 16");
  if (K % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_dgrad_fp8: K must be a multiple of 8");
  if (sge_status st = check_strides("grouped_linear_dgrad_fp8", {N, (int64_t)G * N, hw * 2})) return st;
  if (!aligned16(dy_q) || !aligned16(w_qT) || (dx && !aligned16(dx)) || (preact && !aligned16(preact)) ||
      (dact && !aligned16(dact)))
    return fail(SGE_ERR_ALIGN, "grouped_linear_dgrad_fp8: pointers must be 16-byte aligned");
  const int64_t GN = (int64_t)G * N;
  const Range in[3] = {range_of(dy_q, T, N, N, 1), range_of(w_qT, K, GN, GN, 1),
                       swiglu ? range_of(preact, T, hw, hw, 2) : Range{0, 0}};
  const Range out = swiglu ? range_of(dact, T, hw, hw, 2) : range_of(dx, T, K, K, 2);
  const Range ram = dact_amax ? range_of(dact_amax, 1, G, G, 4) : Range{0, 0};
  for (const Range& i : in)
    if (overlap(out, i) || overlap(ram, i)) return fail(SGE_ERR_ALIAS, "grouped_linear_dgrad_fp8: output overlaps an input");
  if (overlap(out, ram)) return fail(SGE_ERR_ALIAS, "grouped_linear_dgrad_fp8: outputs overlap");
  const size_t need = sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue);
  if (need && (!workspace || workspace_bytes < need))
    return fail(SGE_ERR_WORKSPACE, "grouped_linear_dgrad_fp8: workspace %zu < %zu bytes", workspace_bytes, need);
  if (dact_amax) {
    const hipError_t z = sge::launch_fill_f32_zero(dact_amax, G, stream);
    if (z != hipSuccess) return hip_status(z, "amax fill");
  }
  if (T == 0 || K == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dy_q);
  p.lda = N;
  p.b = static_cast<const uint8_t*>(w_qT);       // the transposed copy [K][G*N], group g at column g*N
  p.ldb = GN;
  p.M = T;
  p.N = K;
  p.K = N;
  p.b_group_stride = N;
  p.a_sinv = dy_sinv;
  p.b_sinv = w_sinv;
  p.sinv_per_group = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(swiglu ? nullptr : dx);
  p.ldc = K;
  p.offsets = offsets;
  p.G = G;
  p.T = T;
  if (swiglu) {
    p.probs = probs;
    p.aux = const_cast<uint16_t*>(static_cast<const uint16_t*>(preact));
    p.ld_aux = hw;
    p.aux_out = static_cast<uint16_t*>(dact);
    p.ld_aux_out = hw;
    p.dp_part = static_cast<float*>(workspace);
    p.F = K;
    p.amax_out = dact_amax;
  }
  set_act(p, epilogue, act_params);
  hipError_t e = sge::launch_grouped_dgrad_fp8(p, epilogue, stream);
  if (e != hipSuccess) return hip_status(e, "grouped dgrad fp8 launch");
  if (swiglu) {
    const int parts = (int)(sge::gemm_dp_parts_per_tile() * ((K + sge::gemm_tile_n() - 1) / sge::gemm_tile_n()));
    e = sge::launch_rowsum_parts(static_cast<const float*>(workspace), parts, offsets, G, T, dprobs, stream);
    if (e != hipSuccess) return hip_status(e, "dprobs reduction launch");
  }
  return ok();
}

sge_status sge_grouped_linear_wgrad_fp8(const void* dyT_q, const float* dy_sinv, const void* xT_q, const float* x_sinv,
                                        int32_t G, int64_t N, int64_t K, const int64_t* layout, int64_t ld,
                                        float alpha, void* dw, hipStream_t stream) {
  if (G < 1 || G > 4096 || N < 0 || K < 0 || ld < 0) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_fp8: bad sizes");
  if (!dyT_q || !dy_sinv || !xT_q || !x_sinv || !layout || !dw) return fail(SGE_ERR_NULL, "grouped_linear_wgrad_fp8: NULL pointer");
  if (ld % SGE_MX_TOKEN_ALIGN) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_fp8: ld must be a multiple of %d", SGE_MX_TOKEN_ALIGN);
  if (K % 8) return fail(SGE_ERR_SHAPE, "grouped_linear_wgrad_fp8: K must be a multiple of 8");
  if (sge_status st = check_strides("grouped_linear_wgrad_fp8", {ld, K * 2})) return st;
  if (!aligned16(dyT_q) || !aligned16(xT_q) || !aligned16(dw))
    return fail(SGE_ERR_ALIGN, "grouped_linear_wgrad_fp8: pointers must be 16-byte aligned");
  const Range rdw = range_of(dw, (int64_t)G * N, K, K, 2);
  const Range in[3] = {range_of(dyT_q, N, ld, ld, 1), range_of(xT_q, K, ld, ld, 1),
                       Range{(uintptr_t)layout, (uintptr_t)(layout + 2 * (G + 1))}};
  for (const Range& i : in)
    if (overlap(rdw, i)) return fail(SGE_ERR_ALIAS, "grouped_linear_wgrad_fp8: dw overlaps an input");
  if (N == 0 || K == 0) return ok();
  sge::GemmParams p;
  memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dyT_q);
  p.lda = ld;
  p.b = static_cast<const uint8_t*>(xT_q);
  p.ldb = ld;
  p.M = N;
  p.N = K;
  p.K = ld;
  p.a_sinv = dy_sinv;
  p.b_sinv = x_sinv;
  p.sinv_per_group = 1;
  p.alpha = alpha;
  p.c = static_cast<uint16_t*>(dw);
  p.ldc = K;
  p.c_group_stride = N * K;
  p.offsets = layout + G + 1;                    // the aligned group starts: each group's contraction range
  p.G = G;
  p.T = ld;
  return hip_status(sge::launch_grouped_wgrad_fp8(p, stream), "grouped wgrad fp8 launch");
}

size_t sge_norm_fwd_workspace_size(int64_t rows, int64_t cols) {
  (void)cols;
  return rows < 0 ? 0 : (size_t)sge::norm_blocks(rows) * 4;
}

sge_status sge_norm_fwd(int32_t kind, const void* x, const void* gamma, const void* beta, int64_t rows, int64_t cols,
                        float eps, int32_t zero_centered, void* y, float* mu, float* rsigma, uint8_t* q, uint8_t* q_t,
                        float* amax, float* scale, float* scale_inv, uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT,
                        uint8_t* s_colT, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kind != SGE_NORM_RMS && kind != SGE_NORM_LAYER) return fail(SGE_ERR_ARG, "norm_fwd: kind %d unknown", kind);
  const bool ln = kind == SGE_NORM_LAYER;
  if (rows < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "norm_fwd: negative size");
  // per-row pointers may be NULL when there are no rows
  if (!gamma || (ln && !beta) || (rows > 0 && (!x || !y || !rsigma || (ln && !mu))))
    return fail(SGE_ERR_NULL, "norm_fwd: NULL pointer");
  const bool fp8 = q || q_t, mxr = q_row || s_row, mxc = q_colT || s_colT;
  if (fp8 && (!amax || !scale || !scale_inv))
    return fail(SGE_ERR_NULL, "norm_fwd: the FP8 output needs amax, scale and scale_inv");
  if ((mxr && (!q_row || !s_row)) || (mxc && (!q_colT || !s_colT)))
    return fail(SGE_ERR_NULL, "norm_fwd: MXFP8 data and scale pointers come in pairs");
  if (cols == 0 || cols % 8 || cols > 16384) return fail(SGE_ERR_SHAPE, "norm_fwd: cols must be a multiple of 8 in [8, 16384]");
  if ((mxr || mxc) && cols % 32) return fail(SGE_ERR_SHAPE, "norm_fwd: MXFP8 output needs cols %% 32 == 0");
  if (mxc && rows % 32) return fail(SGE_ERR_SHAPE, "norm_fwd: the columnwise MXFP8 copy needs rows %% 32 == 0");
  if (fp8 && (rows % 16 || cols % 16)) return fail(SGE_ERR_SHAPE, "norm_fwd: FP8 output needs rows and cols %% 16 == 0");
  if ((x && !aligned16(x)) || !aligned16(gamma) || (beta && !aligned16(beta)) || (y && !aligned16(y)) || (q && !aligned16(q)) ||
      (q_t && !aligned16(q_t)) || (q_row && !aligned16(q_row)) || (q_colT && !aligned16(q_colT)))
    return fail(SGE_ERR_ALIGN, "norm_fwd: pointers must be 16-byte aligned");
  const Range in[3] = {range_of(x, rows, cols, cols, 2), range_of(gamma, 1, cols, cols, 2),
                       ln ? range_of(beta, 1, cols, cols, 2) : Range{0, 0}};
  const Range outs[9] = {range_of(y, rows, cols, cols, 2), ln ? range_of(mu, 1, rows, rows, 4) : Range{0, 0},
                         range_of(rsigma, 1, rows, rows, 4), q ? range_of(q, rows, cols, cols, 1) : Range{0, 0},
                         q_t ? range_of(q_t, cols, rows, rows, 1) : Range{0, 0},
                         q_row ? range_of(q_row, rows, cols, cols, 1) : Range{0, 0},
                         s_row ? range_of(s_row, rows, cols / 32, cols / 32, 1) : Range{0, 0},
                         q_colT ? range_of(q_colT, cols, rows, rows, 1) : Range{0, 0},
                         s_colT ? range_of(s_colT, cols, rows / 32, rows / 32, 1) : Range{0, 0}};
  for (int a = 0; a < 9; ++a) {
    for (const Range& i : in)
      if (overlap(outs[a], i)) return fail(SGE_ERR_ALIAS, "norm_fwd: an output overlaps an input");
    for (int b = a + 1; b < 9; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "norm_fwd: outputs overlap");
  }
  const size_t need = fp8 ? sge_norm_fwd_workspace_size(rows, cols) : 0;
  if (need && (!workspace || workspace_bytes < need))
    return fail(SGE_ERR_WORKSPACE, "norm_fwd: workspace %zu < %zu bytes", workspace_bytes, need);
  if (rows == 0) return ok();
  uint32_t* part = fp8 ? static_cast<uint32_t*>(workspace) : nullptr;
  hipError_t e = sge::launch_norm_fwd(ln, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                                      static_cast<const uint16_t*>(beta), rows, cols, eps, zero_centered ? 1 : 0,
                                      static_cast<uint16_t*>(y), ln ? mu : nullptr, rsigma, part, q_row, s_row, stream);
  if (e != hipSuccess) return hip_status(e, "norm_fwd launch");
  if (fp8) {
    e = sge::launch_quantize_fp8(static_cast<const uint16_t*>(y), rows, cols, part, sge::norm_blocks(rows), q, q_t,
                                 amax, scale, scale_inv, stream);
    if (e != hipSuccess) return hip_status(e, "norm_fwd quantize launch");
  }
  if (mxc) {
    e = sge::launch_quantize_mxfp8(static_cast<const uint16_t*>(y), rows, cols, nullptr, nullptr, q_colT, s_colT,
                                   stream);
    if (e != hipSuccess) return hip_status(e, "norm_fwd columnwise MXFP8 launch");
  }
  return ok();
}

size_t sge_norm_bwd_workspace_size(int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return 0;
  return (size_t)sge::norm_bwd_blocks(rows) * (size_t)cols * 2 * sizeof(float);
}

sge_status sge_norm_bwd(int32_t kind, const void* dz, const void* x, const float* mu, const float* rsigma,
                        const void* gamma, int64_t rows, int64_t cols, int32_t zero_centered, void* dx, void* dgamma,
                        void* dbeta, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (kind != SGE_NORM_RMS && kind != SGE_NORM_LAYER) return fail(SGE_ERR_ARG, "norm_bwd: kind %d unknown", kind);
  const bool ln = kind == SGE_NORM_LAYER;
  if (rows < 0 || cols < 0) return fail(SGE_ERR_SHAPE, "norm_bwd: negative size");
  // per-row pointers may be NULL when there are no rows
  if (!gamma || !dgamma || (ln && !dbeta) || (rows > 0 && (!dz || !x || !rsigma || !dx || (ln && !mu))))
    return fail(SGE_ERR_NULL, "norm_bwd: NULL pointer");
  if (cols == 0 || cols % 8 || cols > 16384) return fail(SGE_ERR_SHAPE, "norm_bwd: cols must be a multiple of 8 in [8, 16384]");
  if ((dz && !aligned16(dz)) || (x && !aligned16(x)) || !aligned16(gamma) || (dx && !aligned16(dx)))
    return fail(SGE_ERR_ALIGN, "norm_bwd: pointers must be 16-byte aligned");
  const Range in[5] = {range_of(dz, rows, cols, cols, 2), range_of(x, rows, cols, cols, 2),
                       range_of(gamma, 1, cols, cols, 2), range_of(rsigma, 1, rows, rows, 4),
                       ln ? range_of(mu, 1, rows, rows, 4) : Range{0, 0}};
  const Range outs[3] = {range_of(dx, rows, cols, cols, 2), range_of(dgamma, 1, cols, cols, 2),
                         ln ? range_of(dbeta, 1, cols, cols, 2) : Range{0, 0}};
  for (int a = 0; a < 3; ++a) {
    for (const Range& i : in)
      if (overlap(outs[a], i)) return fail(SGE_ERR_ALIAS, "norm_bwd: an output overlaps an input");
    for (int b = a + 1; b < 3; ++b)
      if (overlap(outs[a], outs[b])) return fail(SGE_ERR_ALIAS, "norm_bwd: outputs overlap");
  }
  const size_t need = sge_norm_bwd_workspace_size(rows, cols);
  if (!workspace || workspace_bytes < need)
    return fail(SGE_ERR_WORKSPACE, "norm_bwd: workspace %zu < %zu bytes", workspace_bytes, need);
  return hip_status(sge::launch_norm_bwd(ln, static_cast<const uint16_t*>(dz), static_cast<const uint16_t*>(x), mu,
                                         rsigma, static_cast<const uint16_t*>(gamma), rows, cols, zero_centered ? 1 : 0,
                                         static_cast<uint16_t*>(dx), static_cast<uint16_t*>(dgamma),
                                         static_cast<uint16_t*>(dbeta), static_cast<float*>(workspace), stream),
                    "norm_bwd launch");
}

sge_status sge_scaled_swiglu_fwd(const void* h, const float* probs, void* y, int64_t T, int64_t F, hipStream_t stream) {
  if (T < 0 || F < 0) return fail(SGE_ERR_SHAPE, "scaled_swiglu_fwd: negative size");
  if (T > 0 && (!h || !probs || !y)) return fail(SGE_ERR_NULL, "scaled_swiglu_fwd: NULL pointer");
  if (F % 8) return fail(SGE_ERR_SHAPE, "scaled_swiglu_fwd: F must be a multiple of 8");
  if ((h && !aligned16(h)) || (y && !aligned16(y))) return fail(SGE_ERR_ALIGN, "scaled_swiglu_fwd: alignment");
  if (T == 0 || F == 0) return ok();
  if (overlap(range_of(y, T, F, F, 2), range_of(h, T, 2 * F, 2 * F, 2)))
    return fail(SGE_ERR_ALIAS, "scaled_swiglu_fwd: y overlaps h");
  return hip_status(sge::launch_swiglu_fwd(static_cast<const uint16_t*>(h), probs, static_cast<uint16_t*>(y), T, F,
                                           stream),
                    "swiglu fwd launch");
}

sge_status sge_scaled_swiglu_bwd(const void* gy, const void* h, const float* probs, void* dh, float* dprobs, int64_t T,
                                 int64_t F, hipStream_t stream) {
  if (T < 0 || F < 0) return fail(SGE_ERR_SHAPE, "scaled_swiglu_bwd: negative size");
  if (T > 0 && (!gy || !h || !probs || !dh || !dprobs)) return fail(SGE_ERR_NULL, "scaled_swiglu_bwd: NULL pointer");
  if (F % 8) return fail(SGE_ERR_SHAPE, "scaled_swiglu_bwd: F must be a multiple of 8");
  if ((gy && !aligned16(gy)) || (h && !aligned16(h)) || (dh && !aligned16(dh)))
    return fail(SGE_ERR_ALIGN, "scaled_swiglu_bwd: alignment");
  if (T == 0) return ok();
  const Range rdh = range_of(dh, T, 2 * F, 2 * F, 2);
  if (overlap(rdh, range_of(h, T, 2 * F, 2 * F, 2)) || overlap(rdh, range_of(gy, T, F, F, 2)))
    return fail(SGE_ERR_ALIAS, "scaled_swiglu_bwd: dh overlaps an input");
  return hip_status(sge::launch_swiglu_bwd(static_cast<const uint16_t*>(gy), static_cast<const uint16_t*>(h), probs,
                                           static_cast<uint16_t*>(dh), dprobs, T, F, stream),
                    "swiglu bwd launch");
}

// ------------------------------------------------------------------ grouped MLP
// fc1 -> scaled activation -> fc2 as one call each way, chaining the grouped-linear calls above.
// Every argument is checked here, before the first launch, so a rejected call enqueues nothing.
struct Arg {
  Range r;
  unsigned align;   // required alignment of the base pointer in bytes
};

static sge_status check_mlp(const char* what, int32_t G, int64_t T, int64_t H, int64_t F, int32_t activation,
                            const sge_act_params* act_params, const void* const* need, int n_need, const Arg* ins,
                            int n_in, const Arg* outs, int n_out) {
  if (G < 1 || T < 0 || H <= 0 || F <= 0) return fail(SGE_ERR_SHAPE, "%s: bad sizes", what);
  if (activation != SGE_EPI_SCALED_SWIGLU && activation != SGE_EPI_SCALED_SRELU &&
      activation != SGE_EPI_SCALED_CLAMPED_SWIGLU)
    return fail(SGE_ERR_ARG, "%s: activation %d not allowed", what, activation);
  if (sge_status st = check_act(activation, act_params, what)) return st;
  for (int i = 0; i < n_need; ++i)
    if (!need[i])
      return fail(SGE_ERR_NULL, "%s: a required pointer is NULL (W1, W2, offsets, or a T-sized tensor)", what);
  if (H % 8 || F % 8) return fail(SGE_ERR_SHAPE, "%s: H and F must be multiples of 8", what);
  if (gated_fwd(activation) && F % 128) return fail(SGE_ERR_SHAPE, "%s: a gated activation needs F %% 128 == 0", what);
  const int64_t N1 = gated_fwd(activation) ? 2 * F : F;
  if (sge_status st = check_strides(what, {H * 2, N1 * 2})) return st;
  if (gated_fwd(activation))
    if (sge_status st = check_span(what, (F + 256) * H * 2)) return st;
  for (int i = 0; i < n_in + n_out; ++i) {
    const Arg& a = i < n_in ? ins[i] : outs[i - n_in];
    if (a.r.lo % a.align) return fail(SGE_ERR_ALIGN, "%s: argument not %u-byte aligned", what, a.align);
  }
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i].r, ins[j].r)) return fail(SGE_ERR_ALIAS, "%s: an output overlaps an input", what);
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i].r, outs[j].r)) return fail(SGE_ERR_ALIAS, "%s: outputs overlap", what);
  }
  return SGE_OK;
}

sge_status sge_grouped_mlp_fwd(const void* x, const void* w1, const void* w2, int32_t G, int64_t T, int64_t H,
                               int64_t F, const int64_t* splits, int64_t* offsets, int32_t* err_flag,
                               int32_t activation, const sge_act_params* act_params, const float* probs,
                               void* preact, void* act_out, void* out, hipStream_t stream) {
  const int64_t N1 = gated_fwd(activation) ? 2 * F : F;
  // the T-sized tensors may be NULL (empty) when T == 0
  const void* need[9] = {w1, w2, splits, offsets, T ? x : w1, T ? probs : w1, T ? preact : w1, T ? act_out : w1,
                         T ? out : w1};
  const Arg ins[5] = {{range_of(x, T, H, H, 2), 16}, {range_of(w1, (int64_t)G * N1, H, H, 2), 16},
                      {range_of(w2, (int64_t)G * H, F, F, 2), 16}, {range_of(splits, 1, G, G, 8), 8},
                      {range_of(probs, 1, T, T, 4), 4}};
  const Arg outs[5] = {{range_of(offsets, 1, G + 1, G + 1, 8), 8}, {range_of(preact, T, N1, N1, 2), 16},
                       {range_of(act_out, T, F, F, 2), 16}, {range_of(out, T, H, H, 2), 16},
                       {err_flag ? range_of(err_flag, 1, 1, 1, 4) : Range{0, 0}, 4}};
  if (sge_status st = check_mlp("grouped_mlp_fwd", G, T, H, F, activation, act_params, need, 9, ins, 5, outs, 5))
    return st;
  const int64_t one = 1;
  if (sge_status st = sge_splits_to_offsets(splits, G, &one, 1, T, offsets, err_flag, stream)) return st;
  if (T == 0) return ok();
  if (sge_status st = sge_grouped_linear_fwd(x, w1, G, T, N1, H, offsets, 1.0f, activation, act_params, probs,
                                             act_out, preact, stream))
    return st;
  return sge_grouped_linear_fwd(act_out, w2, G, T, H, F, offsets, 1.0f, SGE_EPI_NONE, nullptr, nullptr, out,
                                nullptr, stream);
}

size_t sge_grouped_mlp_bwd_workspace_size(int64_t T, int64_t F, int32_t G, int32_t activation) {
  const int32_t d = activation == SGE_EPI_SCALED_SWIGLU           ? SGE_EPI_DSCALED_SWIGLU
                    : activation == SGE_EPI_SCALED_SRELU          ? SGE_EPI_DSCALED_SRELU
                    : activation == SGE_EPI_SCALED_CLAMPED_SWIGLU ? SGE_EPI_DSCALED_CLAMPED_SWIGLU
                                                                  : SGE_EPI_NONE;
  return d == SGE_EPI_NONE ? 0 : sge_grouped_linear_bwd_workspace_size(T, F, G, d);
}

sge_status sge_grouped_mlp_bwd(const void* dout, const void* x, const void* w1, const void* w2, int32_t G,
                               int64_t T, int64_t H, int64_t F, const int64_t* offsets, int32_t activation,
                               const sge_act_params* act_params, const float* probs, const void* preact,
                               const void* act_out, void* dpreact, float* dprobs, void* dx, void* dw1, void* dw2,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const int64_t N1 = gated_fwd(activation) ? 2 * F : F;
  // the T-sized tensors may be NULL (empty) when T == 0
  const void* need[10] = {w1, w2, offsets, T ? dout : w1, T ? x : w1, T ? probs : w1, T ? preact : w1,
                          T ? act_out : w1, T ? dpreact : w1, T ? dprobs : w1};
  const Arg ins[8] = {{range_of(dout, T, H, H, 2), 16}, {range_of(x, T, H, H, 2), 16},
                      {range_of(w1, (int64_t)G * N1, H, H, 2), 16}, {range_of(w2, (int64_t)G * H, F, F, 2), 16},
                      {range_of(offsets, 1, G + 1, G + 1, 8), 8}, {range_of(probs, 1, T, T, 4), 4},
                      {range_of(preact, T, N1, N1, 2), 16}, {range_of(act_out, T, F, F, 2), 16}};
  const size_t ws_need = sge_grouped_mlp_bwd_workspace_size(T, F, G, activation);
  const Arg outs[6] = {{range_of(dpreact, T, N1, N1, 2), 16}, {range_of(dprobs, 1, T, T, 4), 4},
                       {dx ? range_of(dx, T, H, H, 2) : Range{0, 0}, 16},
                       {dw1 ? range_of(dw1, (int64_t)G * N1, H, H, 2) : Range{0, 0}, 16},
                       {dw2 ? range_of(dw2, (int64_t)G * H, F, F, 2) : Range{0, 0}, 16},
                       {workspace ? range_of(workspace, 1, (int64_t)ws_need, (int64_t)ws_need, 1) : Range{0, 0}, 4}};
  if (sge_status st = check_mlp("grouped_mlp_bwd", G, T, H, F, activation, act_params, need, 10, ins, 8, outs, 6))
    return st;
  if (workspace_bytes < ws_need || (ws_need && !workspace))
    return fail(SGE_ERR_WORKSPACE, "grouped_mlp_bwd: workspace %zu bytes, need %zu", workspace_bytes, ws_need);
  if (T == 0) {                                          // empty groups: zero weight gradients
    hipError_t e = hipSuccess;
    if (dw2) e = sge::launch_fill_bf16_zero(static_cast<uint16_t*>(dw2), (int64_t)G * H, F, F, stream);
    if (e == hipSuccess && dw1)
      e = sge::launch_fill_bf16_zero(static_cast<uint16_t*>(dw1), (int64_t)G * N1, H, H, stream);
    return hip_status(e, "grouped_mlp_bwd fill");
  }
  const int32_t dact = activation == SGE_EPI_SCALED_SWIGLU  ? SGE_EPI_DSCALED_SWIGLU
                       : activation == SGE_EPI_SCALED_SRELU ? SGE_EPI_DSCALED_SRELU
                                                            : SGE_EPI_DSCALED_CLAMPED_SWIGLU;
  // fc2: dgrad through the activation's backward (dpreact, dprobs), and its weight gradient
  if (sge_status st = sge_grouped_linear_bwd(dout, act_out, w2, G, T, H, F, offsets, 1.0f, dact, act_params, preact,
                                             probs, dpreact, dprobs, nullptr, dw2, workspace, workspace_bytes,
                                             stream))
    return st;
  if (!dx && !dw1) return ok();
  // fc1: dgrad and weight gradient from dpreact
  return sge_grouped_linear_bwd(dpreact, x, w1, G, T, N1, H, offsets, 1.0f, SGE_EPI_NONE, nullptr, nullptr, nullptr,
                                nullptr, nullptr, dx, dw1, nullptr, 0, stream);
}

}  // extern "C"
