/*
 * sge.h — C ABI of libsge, the fused scaled linear for AMD Instinct MI355X (gfx950).
 *
 * Every call validates its arguments on the host before any HIP call, then
 * enqueues its kernels on the caller's stream and returns without waiting:
 * no call synchronizes, copies to the host or allocates device memory, so
 * every call can be captured in a HIP graph. Device faults surface at the
 * caller's next synchronization.
 *
 * Ownership: every pointer is caller-owned. Pointers documented "device" must
 * point to device memory of the current device; "host" pointers are read
 * during the call only. Workspaces are sized by the matching *_workspace_size
 * query and passed in by the caller (query, allocate, execute).
 *
 * Errors: a call returns SGE_OK or the first error found, in this order:
 * NULL pointer, shape, format, alignment, aliasing, workspace, then HIP
 * launch errors. sge_last_error_message() gives a thread-local description.
 * On an error before launch nothing was enqueued and no output was touched.
 *
 * Matrices are row-major. A bf16 matrix is stored as 16-bit patterns; an E4M3
 * matrix as bytes (OCP OFP8 E4M3, max 448); an E8M0 scale array as bytes
 * (2^(s-127)). Leading dimensions are in elements. Base pointers must be
 * 16-byte aligned and leading dimensions a multiple of 16 bytes.
 *
 * Size limits: the kernels address a tile (256 rows of a GEMM operand or output, 128 rows of a
 * quantizer's input) through 32-bit byte offsets from the tile's first row, and a few arrays
 * (MXFP8 scale arrays, a gated weight's two halves) from one base. A row stride of more than
 * about 8.3 MB (0x7FFFFF00 / 257 bytes), or such an array of 2^31 bytes or more, gives
 * SGE_ERR_SHAPE rather than being read as zeros.
 */
#ifndef SGE_H
#define SGE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SGE_ABI_VERSION 7

/* Alignment, in tokens, of each group's start in a token-blocked MXFP8 operand. */
#define SGE_MX_TOKEN_ALIGN 128

typedef enum {
  SGE_OK = 0,
  SGE_ERR_NULL = 1,        /* a required pointer is NULL */
  SGE_ERR_SHAPE = 2,       /* negative or inconsistent sizes, or a size the path does not tile */
  SGE_ERR_FORMAT = 3,      /* unknown or unsupported operand format / layout combination */
  SGE_ERR_ALIGN = 4,       /* base pointer or leading dimension not 16-byte aligned */
  SGE_ERR_ALIAS = 5,       /* an output overlaps an input it may not overlap */
  SGE_ERR_WORKSPACE = 6,   /* workspace missing or smaller than the query returned */
  SGE_ERR_ARG = 7,         /* any other invalid argument (flag values, counts) */
  SGE_ERR_HIP = 8          /* a HIP runtime call failed */
} sge_status;

/* Operand formats. */
typedef enum {
  SGE_FMT_BF16 = 0,        /* bf16 values */
  SGE_FMT_E4M3 = 1,        /* E4M3 bytes with one per-tensor fp32 scale_inv (current scaling) */
  SGE_FMT_MXFP8 = 2        /* E4M3 bytes with one E8M0 scale per 32 elements along the contraction dim */
} sge_format;

/*
 * One GEMM operand: a logical matrix [outer, inner] where inner is the
 * dimension the GEMM contracts over.
 *   inner_contiguous = 1: stored as [outer][inner], element (o, i) at data[o*ld + i]
 *   inner_contiguous = 0: stored as [inner][outer], element (o, i) at data[i*ld + o]
 *                          (bf16 only; E4M3/MXFP8 operands are always
 *                          inner-contiguous: the quantizers write the transposed
 *                          copies the backward needs)
 * scale_inv: E4M3 only, device fp32[1] (the value x ~= e4m3(q) * scale_inv).
 * mx_scale:  MXFP8 only, device E8M0 bytes [outer][inner/32] with leading
 *            dimension mx_ld (bytes); element (o, i) is e4m3(q) * 2^(s[o][i/32]-127).
 */
typedef struct {
  const void* data;
  int64_t outer;
  int64_t inner;
  int64_t ld;
  int32_t inner_contiguous;
  int32_t format;              /* sge_format */
  const float* scale_inv;
  const uint8_t* mx_scale;
  int64_t mx_ld;
} sge_operand;

/* Epilogues of the grouped linear. */
typedef enum {
  SGE_EPI_NONE = 0,            /* out = alpha * acc */
  SGE_EPI_SCALED_SWIGLU = 1,   /* forward: h = alpha*acc, y = p * silu(h[:, :F]) * h[:, F:] */
  SGE_EPI_DSCALED_SWIGLU = 2,  /* backward: dgrad g of the next layer -> dh = [da, db], dp */
  SGE_EPI_SCALED_SRELU = 3,    /* forward: h = alpha*acc, y = p * max(h, 0)^2 (elementwise, no gate half) */
  SGE_EPI_DSCALED_SRELU = 4,   /* backward: dh = g * p * 2 max(h, 0), dp = sum_j g * max(h, 0)^2 */
  SGE_EPI_SCALED_CLAMPED_SWIGLU = 5,   /* forward: gated like SWIGLU, clamped (sge_act_params) */
  SGE_EPI_DSCALED_CLAMPED_SWIGLU = 6   /* backward of SCALED_CLAMPED_SWIGLU */
} sge_epilogue;

/*
 * Parameters of the clamped SwiGLU epilogues (host struct, read during the call; NULL for
 * every other epilogue). ("Activation + GroupedLinear Fusion for MOE and other MOE
 * optimizations", Description: scaled SReLU, SwiGLU and clamped SwiGLU activations;
 * Important Files Changed: ScaledClampedQGeGLU. The page names the activation without its
 * formula; this is the published clamped form with the gate through u * sigmoid(alpha * u).)
 * With a, b the two halves of h [T, 2F] and p the per-token scale:
 *   a_c = min(a, limit),  b_c = clamp(b, -limit, limit),
 *   y   = p * a_c * sigmoid(alpha * a_c) * (b_c + 1).
 * Backward (from the saved bf16 h): with s = sigmoid(alpha * a_c), q = a_c * s,
 *   da = g * p * (b_c + 1) * s * (1 + alpha * a_c * (1 - s))  where a <= limit, else 0;
 *   db = g * p * q                                            where |b| <= limit, else 0;
 *   dp = sum_j g_j * q_j * (b_c,j + 1).
 * limit must be finite and > 0 and alpha finite (SGE_ERR_ARG); NULL with a clamped
 * epilogue is SGE_ERR_NULL.
 */
typedef struct {
  float limit;
  float alpha;
} sge_act_params;

int sge_abi_version(void);
const char* sge_status_string(sge_status s);
const char* sge_last_error_message(void);

/*
 * Forward of the fused scaled linear.
 * ("NVIDIA TransformerEngine Ops Fused Forward Linear Scale Add", Description
 * and I/O Contract: the scale is the GEMM alpha and the residual buffer is the
 * GEMM output with accumulation on.)
 *
 *   residual[m][n] <- bf16( (accumulate ? fp32(residual[m][n]) : 0) + alpha_eff * sum_k x[m][k] * w[n][k] )
 *
 * x: operand [M, K] (outer M); w: operand [N, K] (outer N); both the same format.
 * alpha_eff = alpha (BF16, MXFP8) or fp32(fp32(x.scale_inv * w.scale_inv) * alpha) (E4M3).
 * Sums are fp32 (MFMA), rounded once to bf16 (nearest-even).
 * residual: device bf16 [M, N], leading dimension ld_res; read and written in place.
 * alpha == 0: nothing is read or written when accumulate != 0 (the residual is
 * returned bit-exactly); with accumulate == 0 the output is filled with +0.
 * Shapes: K % 8 == 0 (bf16), % 16 (E4M3), % 32 (MXFP8); N % 8 == 0; M >= 0 any.
 * Aliasing: residual may not overlap x or w (SGE_ERR_ALIAS).
 */
sge_status sge_linear_scale_add_fwd(const sge_operand* x, const sge_operand* w, void* residual,
                                    int64_t ld_res, float alpha, int32_t accumulate,
                                    hipStream_t stream);

/*
 * Backward of the fused scaled linear, alpha folded into both GEMMs.
 * ("NVIDIA TransformerEngine Ops Fused Backward Linear Scale", Description and
 * I/O Contract: the scale is passed as grad_input_alpha and grad_weight_alpha.)
 *
 *   dgrad[m][k] = bf16( dgrad_alpha_eff * sum_n dy[m][n] * w[n][k] )     [M, K]
 *   wgrad[n][k] = bf16( wgrad_alpha_eff * sum_m dy[m][n] * x[m][k] )     [N, K]
 *
 * Operands are given in GEMM form (outer, inner = contraction):
 *   dg_a = dy as [M, N]   (bf16: dy itself, inner-contiguous; E4M3/MX: quantized dy)
 *   dg_b = w  as [K, N]   (bf16: w itself with inner_contiguous = 0; E4M3: the
 *                          transposed copy q_t(w) [K][N]; MX: w quantized in blocks along N, stored [K][N])
 *   wg_a = dy as [N, M]   (bf16: dy with inner_contiguous = 0; E4M3/MX: transposed copy [N][M])
 *   wg_b = x  as [K, M]   (bf16: x with inner_contiguous = 0; E4M3/MX: transposed copy [K][M])
 * dgrad / wgrad: device bf16 outputs (overwritten, not accumulated); either may
 * be NULL to skip that GEMM (its operands may then be NULL too).
 * alpha == 0 fills that output with +0 without reading its operands.
 */
sge_status sge_linear_scale_bwd(const sge_operand* dg_a, const sge_operand* dg_b,
                                const sge_operand* wg_a, const sge_operand* wg_b,
                                void* dgrad, int64_t ld_dgrad, void* wgrad, int64_t ld_wgrad,
                                float dgrad_alpha, float wgrad_alpha, hipStream_t stream);

/*
 * FP8 E4M3 per-tensor current scaling of a bf16 matrix [rows, cols].
 * ("NVIDIA TransformerEngine PyTorch Ext Normalization", Description: for
 * current scaling the amax is computed, then the tensor is quantized.)
 *
 *   amax = max |x|;  scale = fp32(448 / amax) (1 if amax == 0, FLT_MAX on overflow);
 *   scale_inv = fp32(1 / scale);  q = e4m3_sat_rne(fp32(x * scale))
 *
 * src: device bf16 [rows][cols] (leading dimension cols).
 * q: device bytes [rows][cols] or NULL; q_t: device bytes [cols][rows] (the
 * transpose) or NULL. amax, scale, scale_inv: device fp32[1] each (required).
 * workspace: device, at least sge_quantize_fp8_amax_workspace_size(rows, cols) bytes.
 * Shapes: rows % 16 == 0 and cols % 16 == 0.
 * Two kernels: a block-wise amax, then a quantize pass that finishes the amax.
 * Non-finite inputs are outside the contract.
 */
size_t sge_quantize_fp8_amax_workspace_size(int64_t rows, int64_t cols);
sge_status sge_quantize_fp8_amax(const void* src, int64_t rows, int64_t cols, uint8_t* q,
                                 uint8_t* q_t, float* amax, float* scale, float* scale_inv,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * sge_quantize_fp8_amax without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * The amax partials go to a scratch array the library holds on each GPU (4 KiB, the most
 * partials the amax pass writes for any tensor size; a size needing more would be refused with
 * SGE_ERR_WORKSPACE). The call allocates nothing. Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams, or host threads) race on it and must be
 * serialized by the caller. Each amax pass writes every partial it later reads, so nothing
 * carries over from an earlier call. Arguments, results and errors are those of
 * sge_quantize_fp8_amax; SGE_ERR_HIP if the array's device address cannot be obtained.
 */
sge_status sge_quantize_fp8_amax_noalloc(const void* src, int64_t rows, int64_t cols, uint8_t* q,
                                         uint8_t* q_t, float* amax, float* scale, float* scale_inv,
                                         hipStream_t stream);

/*
 * MXFP8 quantization of a bf16 matrix [rows, cols], rowwise and/or columnwise.
 * (MXFP8 operands: "core.tensor_parallel.inference_layers", _apply_linear with an
 * MXFP8Tensor; the shared exponent follows OCP MX v1.0 section 6.3.)
 *
 * Per block of 32: X = clamp(floor(log2(max|v|)) - 8, -127, 127) (-127 for an
 * all-zero block), scale byte X + 127, q = e4m3_sat_rne(v * 2^-X).
 * Rowwise: blocks along cols -> q_row [rows][cols], s_row [rows][cols/32].
 * Columnwise: blocks along rows, stored transposed -> q_colT [cols][rows],
 * s_colT [cols][rows/32]. Either pair may be NULL (not both).
 * Shapes: cols % 32 == 0; rows % 32 == 0 when the columnwise copy is requested.
 */
sge_status sge_quantize_mxfp8(const void* src, int64_t rows, int64_t cols, uint8_t* q_row,
                              uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                              hipStream_t stream);

/*
 * Per-group split sizes to tensor offsets, computed once and reused by the
 * forward and the backward.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
 * Description, Precomputed Tensor Offsets Optimization.)
 *
 *   base[0] = 0, base[g+1] = base[g] + splits[g];  offsets[i][g] = base[g] * multipliers[i]
 *
 * splits: device int64 [G]; multipliers: host int64 [n_mult] (1 <= n_mult <= 8);
 * offsets: device int64 [n_mult][G+1]. 1 <= G <= 4096.
 * err_flag: device int32[1] or NULL; when given, it is set to 1 if any split is
 * negative or base[G] != expected_total (pass expected_total < 0 to skip the
 * total check) and to 0 otherwise.
 */
sge_status sge_splits_to_offsets(const int64_t* splits, int32_t G, const int64_t* multipliers,
                                 int32_t n_mult, int64_t expected_total, int64_t* offsets,
                                 int32_t* err_flag, hipStream_t stream);

/*
 * Grouped linear forward over token groups given by device offsets (no host sync).
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
 * Description and Sequence Diagram.)
 *
 * Tokens t in [offsets[g], offsets[g+1]) use weight W_g:
 *   h[t] = alpha * x[t] @ W_g^T                             x [T, K] bf16, W [G, N, K] bf16
 * SGE_EPI_NONE:          out [T, N] bf16 = h.
 * SGE_EPI_SCALED_SWIGLU: F = N/2, a = h[:, :F], b = h[:, F:];
 *                        out [T, F] bf16 = p[t] * silu(a) * b (from the fp32 h),
 *                        preact [T, N] bf16 = h (saved for the backward; may be NULL).
 * SGE_EPI_SCALED_SRELU:  out [T, N] bf16 = p[t] * max(h, 0)^2 (scaled squared ReLU; the page
 *                        names scaled SReLU beside scaled SwiGLU), preact [T, N] = h (or NULL).
 * SGE_EPI_SCALED_CLAMPED_SWIGLU: as SWIGLU with the clamped form of sge_act_params
 *                        (act_params required); preact holds the unclamped h.
 * act_params: host, read during the call; NULL unless the epilogue is clamped.
 * offsets: device int64 [G+1] (row 0 of sge_splits_to_offsets with multiplier 1);
 * values are clamped into [0, T] and made non-decreasing before use.
 * probs: device fp32 [T] (SWIGLU only). Shapes: K % 8 == 0, N % 8 == 0
 * (SWIGLU: N % 256 == 0).
 */
sge_status sge_grouped_linear_fwd(const void* x, const void* w, int32_t G, int64_t T, int64_t N,
                                  int64_t K, const int64_t* offsets, float alpha, int32_t epilogue,
                                  const sge_act_params* act_params,
                                  const float* probs, void* out, void* preact, hipStream_t stream);

/*
 * The whole grouped MLP, fc1 -> scaled activation -> fc2, as one call each way.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations", Description:
 * the offsets are computed once in the forward and reused by the backward; review discussion:
 * the FC1 - ACT - FC2 fused module beside the FC1 - ACT fusion.)
 *
 * A chain of the grouped-linear calls with alpha 1, every argument checked before the first
 * launch (a rejected call enqueues nothing). activation: SGE_EPI_SCALED_SWIGLU,
 * SGE_EPI_SCALED_SRELU or SGE_EPI_SCALED_CLAMPED_SWIGLU (with act_params); N1 = 2F for the
 * gated ones (F % 128 == 0), F for SReLU; H % 8 == 0, F % 8 == 0.
 *
 * sge_grouped_mlp_fwd: splits device int64 [G] -> offsets device int64 [G+1] (exclusive prefix
 *   sum; err_flag, optional device int32, set to 1 when they do not sum to T or one is
 *   negative, else 0), then with x [T, H], W1 [G, N1, H], W2 [G, H, F] (bf16), probs [T] fp32:
 *   preact [T, N1] = h, act_out [T, F] = the scaled activation of h, out [T, H] = fc2 of act_out.
 * sge_grouped_mlp_bwd: from dout [T, H] and the forward's offsets, preact and act_out:
 *   dpreact [T, N1] and dprobs [T] (the activation's backward in fc2's dgrad), dw2 [G, H, F],
 *   dx [T, H], dw1 [G, N1, H] (bf16; dx, dw1, dw2 may each be NULL to skip). workspace: device,
 *   >= sge_grouped_mlp_bwd_workspace_size(T, F, G, activation) bytes.
 * All bf16 tensors 16-byte aligned; outputs may not overlap inputs or each other. With T == 0
 * the T-sized tensors may be NULL: the forward writes the offsets only, the backward zeros
 * dw1 and dw2 (empty sums).
 */
sge_status sge_grouped_mlp_fwd(const void* x, const void* w1, const void* w2, int32_t G, int64_t T,
                               int64_t H, int64_t F, const int64_t* splits, int64_t* offsets,
                               int32_t* err_flag, int32_t activation, const sge_act_params* act_params,
                               const float* probs, void* preact, void* act_out, void* out,
                               hipStream_t stream);
size_t sge_grouped_mlp_bwd_workspace_size(int64_t T, int64_t F, int32_t G, int32_t activation);
sge_status sge_grouped_mlp_bwd(const void* dout, const void* x, const void* w1, const void* w2,
                               int32_t G, int64_t T, int64_t H, int64_t F, const int64_t* offsets,
                               int32_t activation, const sge_act_params* act_params, const float* probs,
                               const void* preact, const void* act_out, void* dpreact, float* dprobs,
                               void* dx, void* dw1, void* dw2, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * Grouped linear forward with MXFP8 operands, and the fused activation + group quantize.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations", Description:
 * Activation + GroupQuantize Fusion, and the forward of the Sequence Diagram, where the
 * scaled activation's output reaches FC2 quantized.)
 *
 * The same computation as sge_grouped_linear_fwd with x and every W_g given as MXFP8
 * quantized rowwise (E4M3 bytes, one E8M0 exponent per 32 elements along K):
 *   x_q [T, K] u8, x_s [T, K/32] u8;  w_q [G, N, K] u8, w_s [G, N, K/32] u8
 *   (exactly what sge_quantize_mxfp8 writes as q_row / s_row).
 * SGE_EPI_NONE: out [T, N] bf16.
 * SGE_EPI_SCALED_SWIGLU: out [T, N/2] bf16 (may be NULL when out_q or out_colT_q is given), preact
 *   [T, N] bf16 (may be NULL), and optionally out_q [T, N/2] u8 + out_s [T, N/64] u8: the
 *   MXFP8 rowwise quantization of the bf16 output, i.e. the bytes sge_quantize_mxfp8 would
 *   write for `out` (the operand layout of the next grouped GEMM's forward). out_q and
 *   out_s are given together or not at all.
 * SGE_EPI_SCALED_SRELU and SGE_EPI_SCALED_CLAMPED_SWIGLU (with act_params) as in
 *   sge_grouped_linear_fwd, with the same optional MXFP8 output.
 * Every activation epilogue may also write the activation output token-blocked (the operand
 *   the next layer's weight gradient contracts over tokens): out_colT_q [C][ld_t] u8 and
 *   out_colT_s [C][ld_t/32] u8 (C = the output's columns; given together, or both NULL),
 *   exactly the q_colT / s_colT that sge_quantize_mxfp8_grouped writes for the bf16 output
 *   with `layout` and ld = ld_t (padding up to each group's aligned end included, columns
 *   from pad[G] on untouched). layout: [2][G+1] from sge_mx_group_layout of the same offsets,
 *   T and G; ld_t % 128 == 0 and ld_t >= sge_mx_token_capacity(T, G). Unused (may be NULL / 0)
 *   without out_colT_q. out may then be NULL.
 * Shapes: K % 128 == 0; N % 8 == 0 (SWIGLU: N % 256 == 0). All pointers 16-byte aligned;
 * outputs must not overlap the inputs or each other (SGE_ERR_ALIAS).
 * offsets and probs as in sge_grouped_linear_fwd.
 */
sge_status sge_grouped_linear_fwd_mxfp8(const void* x_q, const void* x_s, const void* w_q, const void* w_s,
                                        int32_t G, int64_t T, int64_t N, int64_t K, const int64_t* offsets,
                                        float alpha, int32_t epilogue,
                                        const sge_act_params* act_params, const float* probs, void* out,
                                        void* preact, void* out_q, void* out_s, const int64_t* layout,
                                        int64_t ld_t, void* out_colT_q, void* out_colT_s, hipStream_t stream);

/*
 * Grouped linear backward for one layer with the precomputed offsets.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
 * Greptile Summary and Sequence Diagram: the backward reuses the forward's
 * offsets; the activation backward returns the gradient of the scales.)
 *
 * dy [T, N] bf16, x [T, K] bf16 (the layer input), W [G, N, K] bf16.
 *   g[t]  = alpha * dy[t] @ W_g                                      [T, K]
 *   dW_g  = alpha * sum_{t in g} dy[t]^T x[t]                         [G, N, K] (0 for empty groups)
 * SGE_EPI_NONE:           dx [T, K] bf16 = g (dx may be NULL to skip).
 * SGE_EPI_DSCALED_SWIGLU: the layer input x was y = p * silu(a) * b with
 *                         preact h = [a, b] [T, 2K] bf16; writes
 *                         dact [T, 2K] bf16 = [g*p*b*silu'(a), g*p*silu(a)] and
 *                         dprobs [T] fp32 = sum_j g*silu(a)*b (deterministic order).
 *                         dx is not used.
 * SGE_EPI_DSCALED_SRELU:  x was y = p * max(h, 0)^2 with preact h [T, K] bf16; writes
 *                         dact [T, K] = g*p*2*max(h, 0) and dprobs [T] = sum_j g*max(h, 0)^2.
 * SGE_EPI_DSCALED_CLAMPED_SWIGLU: x was the clamped SwiGLU given by act_params (required)
 *                         with preact h = [a, b] [T, 2K] bf16 (unclamped); writes dact [T, 2K]
 *                         and dprobs [T] by the backward given with sge_act_params.
 * dw: device bf16 [G, N, K] or NULL to skip the weight gradient.
 * When both the dgrad (dx or the activation backward) and dw are asked for, the two GEMMs run
 * in one launch (the dgrad's tiles, then the weight gradient's); the results are the same
 * bits as from two calls.
 * workspace: device, >= sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue) bytes
 * (0 is valid for SGE_EPI_NONE).
 */
size_t sge_grouped_linear_bwd_workspace_size(int64_t T, int64_t K, int32_t G, int32_t epilogue);
sge_status sge_grouped_linear_bwd(const void* dy, const void* x, const void* w, int32_t G,
                                  int64_t T, int64_t N, int64_t K, const int64_t* offsets,
                                  float alpha, int32_t epilogue,
                                  const sge_act_params* act_params, const void* preact,
                                  const float* probs, void* dact, float* dprobs, void* dx,
                                  void* dw, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * Token-blocked MXFP8 operands of the grouped weight gradient.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations", Description:
 * the activation is followed by a group quantize, so each group's slice of a grouped tensor
 * is quantized as a tensor of its own; the split offsets are computed once and reused by
 * the backward.)
 *
 * A wgrad contracts over the tokens of one group, so its MXFP8 operands have blocks of 32
 * along tokens, starting at each group's first token; a group whose length is not a
 * multiple of 32 ends in a short block (as if padded with zeros). They are stored
 * transposed, [features][ld], group g from column pad[g], a multiple of SGE_MX_TOKEN_ALIGN:
 *
 *   sge_mx_group_layout: layout [2][G+1] device int64 from offsets [G+1] (device):
 *     layout[0][g] = c[g], the offsets as every grouped call reads them: clamped into [0, T]
 *                    and made non-decreasing (c[g] = max(c[g-1], min(offsets[g], T)), from 0);
 *     layout[1][g] = pad[g]: pad[0] = 0, pad[g+1] = pad[g] + roundup(c[g+1] - c[g], 128).
 *     1 <= G <= 4096. One single-block kernel; computed once, reused by every call below.
 *   sge_mx_token_capacity(T, G): the smallest ld every such operand accepts (an upper
 *     bound of pad[G] known on the host): roundup(T, 128) + 128 * G; -1 for bad sizes.
 *   sge_quantize_mxfp8_grouped: src bf16 [T, cols] (cols % 32 == 0) ->
 *     q_colT [cols][ld] u8 and s_colT [cols][ld/32] u8 (required): token t of group g at
 *     column pad[g] + t - c[g]; columns pad[g] + (c[g+1]-c[g]) .. pad[g+1]-1 hold code 0
 *     under all-zero blocks (E8M0 byte 0); columns from pad[G] on are not written.
 *     Optionally q_row [T, cols] / s_row [T, cols/32] (given together): the rowwise
 *     quantization of sge_quantize_mxfp8, for the tokens inside [c[0], c[G]).
 *     ld % 128 == 0 and ld >= sge_mx_token_capacity(T, G); layout from sge_mx_group_layout
 *     with the same T and G.
 */
int64_t sge_mx_token_capacity(int64_t T, int32_t G);
sge_status sge_mx_group_layout(const int64_t* offsets, int32_t G, int64_t T, int64_t* layout,
                               hipStream_t stream);
sge_status sge_quantize_mxfp8_grouped(const void* src, int64_t T, int64_t cols, int32_t G,
                                      const int64_t* layout, int64_t ld, uint8_t* q_row,
                                      uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT,
                                      hipStream_t stream);

/*
 * Grouped linear backward on MXFP8 operands: the dgrad (with the fused activation backward
 * and group quantize) and the weight gradient.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations", Sequence
 * Diagram, backward: the activation backward hands FC1's dgrad the quantized gradient,
 * FC1's wgrad the same gradient unquantized, and returns the gradient of the scales.)
 *
 * dgrad, for the layer  out[t] = alpha * x[t] @ W_g^T,  W [G, N, K]:
 *   g[t] = alpha * dy[t] @ W_g  (contraction over N, all operands MXFP8 blocked along N)
 *   dy_q [T, N] u8, dy_s [T, N/32] u8: dy quantized rowwise (sge_quantize_mxfp8 q_row/s_row);
 *   w_q [K][G*N] u8, w_s [K][G*N/32] u8: W viewed as [G*N, K] quantized columnwise
 *     (sge_quantize_mxfp8 q_colT/s_colT); blocks never cross experts as N % 32 == 0.
 *   SGE_EPI_NONE: dx [T, K] bf16 = g.
 *   SGE_EPI_DSCALED_SWIGLU (x was y = p * silu(a) * b, preact h = [a, b] [T, 2K] bf16):
 *     dact [T, 2K] bf16 = [g*p*b*silu'(a), g*p*silu(a)] (may be NULL when dact_q or dact_colT_q is given),
 *     dprobs [T] fp32 = sum_j g*silu(a)*b (deterministic order), and optionally
 *     dact_q [T, 2K] u8 + dact_s [T, 2K/32] u8: the rowwise MXFP8 of the bf16 dact, the bytes
 *     sge_quantize_mxfp8 writes for it (the operand of the next layer's dgrad).
 *     workspace: >= sge_grouped_linear_bwd_workspace_size(T, K, G, epilogue) bytes.
 *   SGE_EPI_DSCALED_SRELU and SGE_EPI_DSCALED_CLAMPED_SWIGLU (with act_params) as in
 *   sge_grouped_linear_bwd, with the same optional MXFP8 dact.
 *   With an activation backward, dact may also be written token-blocked (the operand of the
 *   next layer's weight gradient): dact_colT_q [W][ld_t] u8 + dact_colT_s [W][ld_t/32] u8
 *   (W = dact's width; given together), exactly what sge_quantize_mxfp8_grouped writes as
 *   q_colT / s_colT for the bf16 dact with `layout` and ld = ld_t; layout and ld_t as for
 *   sge_grouped_linear_fwd_mxfp8's out_colT_q (unused without dact_colT_q).
 *   Shapes: N % 128 == 0, K % 8 == 0 (SwiGLU: K % 32 == 0). offsets as in
 *   sge_grouped_linear_fwd. Outputs may not overlap inputs or each other.
 *
 * wgrad: dW_g [N, K] bf16 = alpha * sum_{t in g} dy[t]^T x[t], zero for an empty group,
 *   from the token-blocked operands of sge_quantize_mxfp8_grouped:
 *   dyT_q [N][ld], dyT_s [N][ld/32] (of dy [T, N]); xT_q [K][ld], xT_s [K][ld/32] (of the
 *   layer input x [T, K]); layout and ld as given to the quantizer. dw [G, N, K] bf16.
 *   Shapes: ld % 128 == 0, K % 8 == 0, 1 <= G <= 4096.
 */
sge_status sge_grouped_linear_dgrad_mxfp8(const void* dy_q, const void* dy_s, const void* w_q,
                                          const void* w_s, int32_t G, int64_t T, int64_t N, int64_t K,
                                          const int64_t* offsets, float alpha, int32_t epilogue,
                                          const sge_act_params* act_params,
                                          const void* preact, const float* probs, void* dx, void* dact,
                                          float* dprobs, void* dact_q, void* dact_s, const int64_t* layout,
                                          int64_t ld_t, void* dact_colT_q, void* dact_colT_s, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);
sge_status sge_grouped_linear_wgrad_mxfp8(const void* dyT_q, const void* dyT_s, const void* xT_q,
                                          const void* xT_s, int32_t G, int64_t N, int64_t K,
                                          const int64_t* layout, int64_t ld, float alpha, void* dw,
                                          hipStream_t stream);

/*
 * Grouped linear on FP8 E4M3 operands with current scaling per group.
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations", Description:
 * the scaled activation is followed by a group quantize; Greptile Summary: fp8_current_scaling
 * in the grouped-MLP test matrix.) A group quantize gives each group's slice of a grouped
 * tensor (and each expert's weight) a quantizer of its own, so with current scaling every
 * group has its own amax, scale = 448/amax and scale_inv (the per-tensor rules of
 * sge_quantize_fp8_amax, applied group by group).
 *
 * sge_quantize_fp8_grouped: src bf16 [rows, cols] (cols % 16 == 0), groups given either by
 *   layout ([2][G+1] from sge_mx_group_layout: group g owns rows c[g] .. c[g+1]-1) or, with
 *   layout NULL, as G equal runs of rows/G rows (rows/G a multiple of 128: the experts of a
 *   weight viewed [G*N, K]). Writes amax, scale, scale_inv (device fp32 [G] each, required;
 *   an empty group gets 0, 1, 1) and any of:
 *     q   [rows, cols] u8: row r quantized with its group's scale (rows in no group untouched);
 *     q_t [cols][ld_t] u8: the transpose; with a layout, group g's row t at column
 *         pad[g] + t - c[g] and zeros up to pad[g+1] (ld_t % 128 == 0 and
 *         ld_t >= sge_mx_token_capacity(rows, G)); without, column r (ld_t >= rows, ld_t % 16 == 0).
 *   workspace: >= sge_quantize_fp8_grouped_workspace_size(G) bytes. Two kernels: a per-group
 *   amax (atomic max, order-free), then the quantize pass. amax_in (device fp32 [G] or NULL):
 *   the groups' amax already reduced by the producing epilogue (out_amax / dact_amax below);
 *   then only the quantize pass runs (and the workspace may be NULL).
 * sge_grouped_linear_fwd_fp8: as sge_grouped_linear_fwd with x_q [T, K] u8 (x_sinv [G]: the
 *   scale_inv of each group's tokens) and w_q [G, N, K] u8 (w_sinv [G]: each expert's);
 *   h = fp32(x_sinv[g] * w_sinv[g]) * alpha * acc. K % 16 == 0, N % 8 == 0 (SwiGLU N % 256).
 *   out_amax (an activation epilogue only; device fp32 [G] or NULL): each group's amax of the
 *   bf16 output, reduced in the epilogue (the amax a current-scaling quantize of it needs).
 *   Every activation epilogue of sge_grouped_linear_fwd is taken (clamped: with act_params).
 * sge_grouped_linear_dgrad_fp8: as sge_grouped_linear_dgrad_mxfp8 with dy_q [T, N] u8
 *   (dy_sinv [G]) and w_qT [K][G*N] u8, the transpose of W viewed [G*N, K] (the q_t of
 *   sge_quantize_fp8_grouped without a layout; w_sinv [G]). N % 16 == 0, K % 8 == 0; the
 *   SwiGLU backward writes dact [T, 2K] and dprobs [T] (workspace as for sge_grouped_linear_bwd),
 *   and, given dact_amax (device fp32 [G]), each group's amax of the bf16 dact. Every
 *   activation backward of sge_grouped_linear_bwd is taken (clamped: with act_params).
 * sge_grouped_linear_wgrad_fp8: dW_g = fp32(dy_sinv[g] * x_sinv[g]) * alpha * sum_{t in g}
 *   dy[t]^T x[t] from dyT_q [N][ld] and xT_q [K][ld] (q_t with the layout), dw [G, N, K] bf16.
 */
size_t sge_quantize_fp8_grouped_workspace_size(int32_t G);
sge_status sge_quantize_fp8_grouped(const void* src, int64_t rows, int64_t cols, int32_t G,
                                    const int64_t* layout, int64_t ld_t, uint8_t* q, uint8_t* q_t,
                                    float* amax, float* scale, float* scale_inv, const float* amax_in,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream);
sge_status sge_grouped_linear_fwd_fp8(const void* x_q, const float* x_sinv, const void* w_q,
                                      const float* w_sinv, int32_t G, int64_t T, int64_t N, int64_t K,
                                      const int64_t* offsets, float alpha, int32_t epilogue,
                                      const sge_act_params* act_params,
                                      const float* probs, void* out, void* preact, float* out_amax,
                                      hipStream_t stream);
sge_status sge_grouped_linear_dgrad_fp8(const void* dy_q, const float* dy_sinv, const void* w_qT,
                                        const float* w_sinv, int32_t G, int64_t T, int64_t N, int64_t K,
                                        const int64_t* offsets, float alpha, int32_t epilogue,
                                        const sge_act_params* act_params,
                                        const void* preact, const float* probs, void* dx, void* dact,
                                        float* dprobs, float* dact_amax, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream);
sge_status sge_grouped_linear_wgrad_fp8(const void* dyT_q, const float* dy_sinv, const void* xT_q,
                                        const float* x_sinv, int32_t G, int64_t N, int64_t K,
                                        const int64_t* layout, int64_t ld, float alpha, void* dw,
                                        hipStream_t stream);

/*
 * RMSNorm / LayerNorm with the quantized outputs that feed a linear.
 * ("NVIDIA TransformerEngine PyTorch Ext Normalization", Description and I/O Contract: the
 * forward returns the normalized, optionally quantized, output with the statistics saved
 * for the backward; current scaling computes the norm and its amax, then quantizes; MXFP8
 * is written by the norm kernel; the backward returns dx, dgamma and dbeta; gamma may be
 * zero-centered.)
 *
 * x, dz, y, dx: bf16 [rows, cols]; gamma, beta, dgamma, dbeta: bf16 [cols]; mu, rsigma: fp32
 * [rows] (mu LayerNorm only). g = gamma, or 1 + gamma when zero_centered != 0.
 *   RMSNorm:   rsigma = 1/sqrt(mean(x^2) + eps),        y = x * rsigma * g
 *   LayerNorm: mu = mean(x), rsigma = 1/sqrt(mean((x-mu)^2) + eps), y = (x-mu) * rsigma * g + beta
 * Statistics in fp32, y rounded once to bf16 (always written). Optional quantized outputs of
 * the bf16 y, byte-identical to the standalone quantizers run on it:
 *   FP8 current scaling (q [rows, cols] and/or q_t [cols, rows], with amax, scale, scale_inv
 *   as in sge_quantize_fp8_amax): the norm kernel reduces y's amax, a quantize pass follows;
 *   rows % 16 == 0, cols % 16 == 0; workspace >= sge_norm_fwd_workspace_size.
 *   MXFP8 rowwise (q_row [rows, cols] + s_row [rows, cols/32], written by the norm kernel)
 *   and/or columnwise (q_colT [cols, rows] + s_colT [cols, rows/32], a pass over y;
 *   rows % 32 == 0); cols % 32 == 0.
 * Backward (xhat = (x - mu) * rsigma, mu = 0 for RMSNorm, d = dz * g):
 *   dx = rsigma * (d - mean(d) - xhat * mean(d * xhat))   (RMSNorm: without mean(d))
 *   dgamma = sum_rows dz * xhat, dbeta = sum_rows dz (fixed-order sums, deterministic);
 *   mu and rsigma as the forward saved them; workspace >= sge_norm_bwd_workspace_size.
 * cols % 8 == 0 and 8 <= cols <= 16384.
 */
typedef enum { SGE_NORM_RMS = 0, SGE_NORM_LAYER = 1 } sge_norm_kind;
size_t sge_norm_fwd_workspace_size(int64_t rows, int64_t cols);
sge_status sge_norm_fwd(int32_t kind, const void* x, const void* gamma, const void* beta, int64_t rows,
                        int64_t cols, float eps, int32_t zero_centered, void* y, float* mu, float* rsigma,
                        uint8_t* q, uint8_t* q_t, float* amax, float* scale, float* scale_inv,
                        uint8_t* q_row, uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);
size_t sge_norm_bwd_workspace_size(int64_t rows, int64_t cols);
sge_status sge_norm_bwd(int32_t kind, const void* dz, const void* x, const float* mu, const float* rsigma,
                        const void* gamma, int64_t rows, int64_t cols, int32_t zero_centered, void* dx,
                        void* dgamma, void* dbeta, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Unfused per-token scaled SwiGLU (the composition the fused epilogues replace).
 * ("Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
 * Description: scaled SwiGLU tex API.)
 * fwd: y [T, F] = p * silu(h[:, :F]) * h[:, F:]           h [T, 2F] bf16, p [T] fp32
 * bwd: dh [T, 2F] = [gy*p*b*silu'(a), gy*p*silu(a)], dp [T] = sum_j gy*silu(a)*b
 * Shapes: F % 8 == 0.
 */
sge_status sge_scaled_swiglu_fwd(const void* h, const float* probs, void* y, int64_t T, int64_t F,
                                 hipStream_t stream);
sge_status sge_scaled_swiglu_bwd(const void* gy, const void* h, const float* probs, void* dh,
                                 float* dprobs, int64_t T, int64_t F, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SGE_H */
