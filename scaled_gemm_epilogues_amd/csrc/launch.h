// Host-side launch interface between the C ABI (abi.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sge {

// Arguments of one GEMM launch: C[m][n] = epilogue(sum_k A[m][k] * B[n][k]).
// Element strides are in elements of the operand format (2 bytes for bf16,
// 1 byte for E4M3 / MXFP8).
struct GemmParams {
  const uint8_t* a;
  int64_t lda;
  const uint8_t* b;
  int64_t ldb;
  int64_t M, N, K;            // C is [M, N]; K is the contraction length
  int64_t b_group_stride;     // grouped rows: elements from W_g to W_{g+1}
  const float* a_sinv;        // E4M3 per-tensor scale_inv (device fp32[1])
  const float* b_sinv;
  const uint8_t* a_mx;        // MXFP8 E8M0 scales [rows][K/32]
  int64_t a_mx_ld;
  const uint8_t* b_mx;
  int64_t b_mx_ld;
  int mx_aligned;             // K % 128 == 0 and both scale lds % 4 == 0
  float alpha;
  uint16_t* c;
  int64_t ldc;
  int64_t c_group_stride;     // grouped contraction: elements from dW_g to dW_{g+1}
  int accumulate;
  const int64_t* offsets;     // grouped: device int64 [G+1]
  int G;
  int64_t T;
  int mt_count, nt_count;     // filled by the launcher
  const float* probs;         // SwiGLU: per-token scales
  uint16_t* aux;              // SwiGLU fwd: preact out; dSwiGLU: preact in
  int64_t ld_aux;
  uint16_t* aux_out;          // dSwiGLU: dact out
  int64_t ld_aux_out;
  float* dp_part;             // dSwiGLU: per-column-tile partial sums [parts][T]
  int64_t F;                  // SwiGLU half width
  int64_t b_mx_group_stride;  // grouped MXFP8: bytes from W_g's scales to W_{g+1}'s
  uint8_t* q_out;             // SwiGLU with MXFP8 output: E4M3 [T][ld_q] (or NULL)
  uint8_t* s_out;             //   and its E8M0 scales [T][ld_q / 32]
  int64_t ld_q;
  int64_t b_mx_bytes;         // MXFP8: bytes of B's whole scale array from b_mx (0: rows x ld)
  int sinv_per_group;         // E4M3 grouped: a_sinv / b_sinv are [G], indexed by the group
  float* amax_out;            // (d)SwiGLU: per-group amax of the bf16 output, atomic max (zeroed by the caller)
  float act_limit;            // clamped SwiGLU: the clamp bound (gate above, up half both ways)
  float act_alpha;            //   and the gate's sigmoid slope
  // Row-partitioned MXFP8 activation epilogues: the activation output also quantized with
  // blocks of 32 along each group's tokens (the grouped wgrad operand), stored transposed.
  uint8_t* qt_out;            // E4M3 [cols][ld_t], group g's token t at column pad[g] + t - c[g] (or NULL)
  uint8_t* st_out;            //   and its E8M0 scales [cols][ld_t / 32]
  int64_t ld_t;
  const int64_t* mx_layout;   //   [2][G+1]: clamped offsets c, then the 128-aligned group starts pad
};

hipError_t launch_gemm(const GemmParams& p, int fmt, bool a_kmaj, bool b_kmaj, hipStream_t s);
hipError_t launch_grouped_fwd(const GemmParams& p, int epilogue, hipStream_t s);
// The same with MXFP8 operands (scale rows dword-aligned: K % 128 == 0).
hipError_t launch_grouped_fwd_mx(const GemmParams& p, int epilogue, hipStream_t s);
hipError_t launch_grouped_dgrad(const GemmParams& p, int epilogue, hipStream_t s);
hipError_t launch_grouped_wgrad(const GemmParams& p, hipStream_t s);
// The grouped dgrad (epilogue as in launch_grouped_dgrad) and the grouped wgrad of one layer, in
// one launch (the two GEMMs are independent).
hipError_t launch_grouped_dgrad_wgrad(const GemmParams& dg, int epilogue, const GemmParams& wg, hipStream_t s);
// MXFP8 operands, both inner-contiguous (scale rows dword-aligned: contraction % 128 == 0).
hipError_t launch_grouped_dgrad_mx(const GemmParams& p, int epilogue, hipStream_t s);
// E4M3 operands with one scale per group (sinv_per_group), both inner-contiguous.
hipError_t launch_grouped_fwd_fp8(const GemmParams& p, int epilogue, hipStream_t s);
hipError_t launch_grouped_dgrad_fp8(const GemmParams& p, int epilogue, hipStream_t s);
hipError_t launch_grouped_wgrad_fp8(const GemmParams& p, hipStream_t s);
hipError_t launch_grouped_wgrad_mx(const GemmParams& p, hipStream_t s);
int gemm_tile_n();
int gemm_dp_parts_per_tile();

hipError_t launch_fill_bf16_zero(uint16_t* c, int64_t rows, int64_t cols, int64_t ld, hipStream_t s);
hipError_t launch_fill_f32_zero(float* c, int64_t n, hipStream_t s);

hipError_t launch_amax_partial(const uint16_t* src, int64_t n, uint32_t* partial, int nblocks,
                               hipStream_t s);
int amax_partial_blocks(int64_t n);
// Device address and size of this GPU's amax partial scratch array (no allocation; the address is
// looked up once per device, with that device current).
hipError_t amax_scratch(uint32_t** partial, size_t* bytes);
hipError_t launch_quantize_fp8(const uint16_t* src, int64_t rows, int64_t cols, const uint32_t* partial,
                               int nparts, uint8_t* q, uint8_t* q_t, float* amax, float* scale,
                               float* scale_inv, hipStream_t s);
hipError_t launch_quantize_mxfp8(const uint16_t* src, int64_t rows, int64_t cols, uint8_t* q_row,
                                 uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, hipStream_t s);
// Token-blocked (per group) MXFP8: layout = [clamped offsets; aligned starts], [2][G+1].
hipError_t launch_quantize_mxfp8_grouped(const uint16_t* src, int64_t rows, int64_t cols, int G,
                                         const int64_t* layout, int64_t ld_t, uint8_t* q_row, uint8_t* s_row,
                                         uint8_t* q_colT, uint8_t* s_colT, hipStream_t s);
// FP8 current scaling with one scale per group (layout NULL: G equal runs of rows / G rows).
hipError_t launch_quantize_fp8_grouped(const uint16_t* src, int64_t rows, int64_t cols, int G,
                                       const int64_t* layout, int64_t ld_t, float* amax_ws, const float* amax_in,
                                       uint8_t* q, uint8_t* q_t, float* amax, float* scale, float* scale_inv,
                                       hipStream_t s);
hipError_t launch_mx_group_layout(const int64_t* offsets, int G, int64_t T, int64_t align, int64_t* layout,
                                  hipStream_t s);

// RMSNorm (ln false) / LayerNorm forward: bf16 y, fp32 mu (LayerNorm; may be NULL) and rsigma
// per row; optionally one amax partial per block (norm_blocks(rows) of them) and the rowwise
// MXFP8 copy of y. cols % 32 == 0 (8 for no MXFP8), cols <= 16384.
int norm_blocks(int64_t rows);
int norm_bwd_blocks(int64_t rows);
hipError_t launch_norm_fwd(bool ln, const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                           int64_t cols, float eps, int zc, uint16_t* y, float* mu, float* rsigma,
                           uint32_t* amax_part, uint8_t* q_row, uint8_t* s_row, hipStream_t s);
// Backward: dx bf16, dgamma (and LayerNorm dbeta) bf16 [cols] via fp32 partials
// [2][norm_bwd_blocks(rows)][cols] in `part`.
hipError_t launch_norm_bwd(bool ln, const uint16_t* dz, const uint16_t* x, const float* mu, const float* rsigma,
                           const uint16_t* gamma, int64_t rows, int64_t cols, int zc, uint16_t* dx, uint16_t* dgamma,
                           uint16_t* dbeta, float* part, hipStream_t s);
hipError_t launch_splits_to_offsets(const int64_t* splits, int G, const int64_t* mults, int n_mult,
                                    int64_t expected_total, int64_t* offsets, int32_t* err_flag,
                                    hipStream_t s);
hipError_t launch_swiglu_fwd(const uint16_t* h, const float* p, uint16_t* y, int64_t T, int64_t F,
                             hipStream_t s);
hipError_t launch_swiglu_bwd(const uint16_t* gy, const uint16_t* h, const float* p, uint16_t* dh,
                             float* dp, int64_t T, int64_t F, hipStream_t s);
hipError_t launch_rowsum_parts(const float* part, int nparts, const int64_t* offsets, int G, int64_t T,
                               float* out, hipStream_t s);

}  // namespace sge
