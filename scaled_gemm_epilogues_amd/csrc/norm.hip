// RMSNorm and LayerNorm for gfx950, forward and backward, with the quantized outputs that feed
// a linear ("NVIDIA TransformerEngine PyTorch Ext Normalization", Description and I/O
// Contract: the forward returns the normalized, optionally quantized, output and the saved
// statistics; with current scaling the norm computes its amax and a quantize pass follows;
// MXFP8 is produced by the norm kernel itself; the backward returns dx, dgamma, dbeta).
//
// Forward: one row per block iteration (grid-stride over rows, at most kNormBlocks blocks),
// 256 threads, thread t owning the 8-column chunks 8t + 2048i. Statistics in fp32 with a
// fixed-order block reduction (LayerNorm's variance in a second pass around the mean); the
// output is rounded once to bf16. With AMAX each block also reduces the bf16 output's
// magnitude into one partial (the current-scaling quantize pass finishes it); with MXROW the
// rowwise MXFP8 copy of the bf16 output is written from registers (four adjacent lanes hold a
// 32-column block), the bytes the standalone quantizer writes for the same bf16 output.
//
// Backward: the same row walk with the row's dz and x held in registers (one HBM read each);
// per row the two means (of d*xhat, and of d for LayerNorm) are block-reduced, dx is written
// in bf16, and each block keeps its own column sums of dz*xhat and dz in registers, stored
// once as fp32 partials; a second kernel adds the partials of all blocks in a fixed order
// (deterministic dgamma / dbeta).
#include "common.h"
#include "launch.h"

namespace sge {

constexpr int kNormThreads = 256;
constexpr int kNormBlocks = 1024;        // forward grid cap (= amax partials the quantize pass reduces)
constexpr int kNormBwdBlocks = 512;      // backward grid cap (= dgamma / dbeta partial rows)

__device__ __forceinline__ float block_sum_f32(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();                                       // red[] free from the previous use
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float s = 0.0f;
#pragma unroll
  for (int w = 0; w < kNormThreads / 64; ++w) s += red[w];
  return s;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_lo(w[e]);
    v[2 * e + 1] = bf16_hi(w[e]);
  }
}

template <bool LN, bool AMAX, bool MXROW>
__global__ __launch_bounds__(kNormThreads) void norm_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ beta,
    int64_t rows, int64_t cols, float eps, int zero_centered, uint16_t* __restrict__ y, float* __restrict__ mu_out,
    float* __restrict__ rsigma_out, uint32_t* __restrict__ amax_part, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row) {
  __shared__ float red[kNormThreads / 64];
  const int t = threadIdx.x;
  const int nch = (int)((cols / 8 + kNormThreads - 1) / kNormThreads);   // uniform over the block
  const float gofs = zero_centered ? 1.0f : 0.0f;
  const float inv_cols = 1.0f / (float)cols;
  uint32_t amax = 0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint16_t* xr = x + r * cols;
    float mu = 0.0f;
    if constexpr (LN) {
      float s = 0.0f;
      for (int i = 0; i < nch; ++i) {
        const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
        if (c < cols) {
          float v[8];
          load8(xr + c, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) s += v[e];
        }
      }
      mu = block_sum_f32(s, red) * inv_cols;
    }
    float ss = 0.0f;
    for (int i = 0; i < nch; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      if (c < cols) {
        float v[8];
        load8(xr + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = v[e] - mu;
          ss += d * d;
        }
      }
    }
    const float rs = 1.0f / sqrtf(block_sum_f32(ss, red) * inv_cols + eps);
    for (int i = 0; i < nch; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      const bool ok = c < cols;
      v4i vy = {0, 0, 0, 0};
      if (ok) {
        float v[8], g[8], b[8];
        load8(xr + c, v);
        load8(gamma + c, g);
        if constexpr (LN) load8(beta + c, b);
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = (v[e] - mu) * rs * (g[e] + gofs);
          if constexpr (LN) o[e] += b[e];
        }
        vy = v4i{(int)pack_bf16x2(o[0], o[1]), (int)pack_bf16x2(o[2], o[3]), (int)pack_bf16x2(o[4], o[5]),
                 (int)pack_bf16x2(o[6], o[7])};
        *reinterpret_cast<v4i*>(y + r * cols + c) = vy;
        if constexpr (AMAX) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = (uint32_t)vy[e], lo = w & 0x7FFFu, hi = (w >> 16) & 0x7FFFu;
            amax = lo > amax ? lo : amax;
            amax = hi > amax ? hi : amax;
          }
        }
      }
      if constexpr (MXROW) {
        int e8;
        const v2i qv = mx_quant_lane8(vy, e8);                // every lane takes part
        if (ok) {
          *reinterpret_cast<v2i*>(q_row + r * cols + c) = qv;
          if ((t & 3) == 0) s_row[r * (cols / 32) + c / 32] = (uint8_t)e8;
        }
      }
    }
    if (t == 0) {
      if (mu_out) mu_out[r] = mu;
      rsigma_out[r] = rs;
    }
  }
  if constexpr (AMAX) {
    amax = wave_max(amax);
    const int lane = t & 63, wave = t >> 6;
    __shared__ uint32_t redm[kNormThreads / 64];
    if (lane == 0) redm[wave] = amax;
    __syncthreads();
    if (t == 0) {
      uint32_t m = 0;
      for (int w = 0; w < kNormThreads / 64; ++w) m = redm[w] > m ? redm[w] : m;
      amax_part[blockIdx.x] = m;
    }
  }
}

template <bool LN, int NCH>
__global__ __launch_bounds__(kNormThreads) void norm_bwd_kernel(
    const uint16_t* __restrict__ dz, const uint16_t* __restrict__ x, const float* __restrict__ mu_in,
    const float* __restrict__ rsigma_in, const uint16_t* __restrict__ gamma, int64_t rows, int64_t cols,
    int zero_centered, uint16_t* __restrict__ dx, float* __restrict__ dg_part, float* __restrict__ db_part) {
  // NCH: chunks of 8 columns per thread (cols <= 2048 * NCH); the row's dz and x stay in
  // registers (as loaded bf16) between the reduction pass and the dx pass.
  __shared__ float red[kNormThreads / 64];
  const int t = threadIdx.x;
  const float gofs = zero_centered ? 1.0f : 0.0f;
  const float inv_cols = 1.0f / (float)cols;
  float pg[NCH][8], pb[NCH][8], g[NCH][8];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
#pragma unroll
    for (int e = 0; e < 8; ++e) pg[i][e] = pb[i][e] = g[i][e] = 0.0f;
    if (c < cols) {
      load8(gamma + c, g[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) g[i][e] += gofs;
    }
  }
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const float rs = rsigma_in[r];
    const float m = LN ? mu_in[r] : 0.0f;
    const uint16_t* dzr = dz + r * cols;
    const uint16_t* xr = x + r * cols;
    uint4 ud[NCH], ux[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      ud[i] = ux[i] = make_uint4(0, 0, 0, 0);
      if (c < cols) {
        ud[i] = *reinterpret_cast<const uint4*>(dzr + c);
        ux[i] = *reinterpret_cast<const uint4*>(xr + c);
      }
    }
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const uint32_t wd[4] = {ud[i].x, ud[i].y, ud[i].z, ud[i].w}, wx[4] = {ux[i].x, ux[i].y, ux[i].z, ux[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]);
        const float v = (e & 1) ? bf16_hi(wx[e >> 1]) : bf16_lo(wx[e >> 1]);
        const float xh = (v - m) * rs;
        const float dg = d * g[i][e];
        s1 += dg * xh;
        if constexpr (LN) s2 += dg;
        pg[i][e] += d * xh;                              // zero for columns past the row (d = 0)
        if constexpr (LN) pb[i][e] += d;
      }
    }
    const float m1 = block_sum_f32(s1, red) * inv_cols;
    const float m2 = LN ? block_sum_f32(s2, red) * inv_cols : 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      if (c < cols) {
        const uint32_t wd[4] = {ud[i].x, ud[i].y, ud[i].z, ud[i].w}, wx[4] = {ux[i].x, ux[i].y, ux[i].z, ux[i].w};
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = (e & 1) ? bf16_hi(wd[e >> 1]) : bf16_lo(wd[e >> 1]);
          const float v = (e & 1) ? bf16_hi(wx[e >> 1]) : bf16_lo(wx[e >> 1]);
          const float xh = (v - m) * rs;
          o[e] = rs * (d * g[i][e] - m2 - xh * m1);
        }
        *reinterpret_cast<v4i*>(dx + r * cols + c) =
            v4i{(int)pack_bf16x2(o[0], o[1]), (int)pack_bf16x2(o[2], o[3]), (int)pack_bf16x2(o[4], o[5]),
                (int)pack_bf16x2(o[6], o[7])};
      }
    }
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
    if (c < cols) {
      float* dg = dg_part + (int64_t)blockIdx.x * cols + c;
#pragma unroll
      for (int e = 0; e < 8; ++e) dg[e] = pg[i][e];
      if constexpr (LN) {
        float* db = db_part + (int64_t)blockIdx.x * cols + c;
#pragma unroll
        for (int e = 0; e < 8; ++e) db[e] = pb[i][e];
      }
    }
  }
}

// out[c] = bf16(sum over parts b, in order, of part[b][c]).
__global__ __launch_bounds__(256) void colsum_parts_kernel(const float* __restrict__ part, int nparts, int64_t cols,
                                                          uint16_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int b = 0; b < nparts; ++b) s += part[(int64_t)b * cols + c];
  out[c] = f32_to_bf16(s);
}

int norm_blocks(int64_t rows) { return (int)(rows < kNormBlocks ? (rows < 1 ? 1 : rows) : kNormBlocks); }
int norm_bwd_blocks(int64_t rows) { return (int)(rows < kNormBwdBlocks ? (rows < 1 ? 1 : rows) : kNormBwdBlocks); }

hipError_t launch_norm_fwd(bool ln, const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                           int64_t cols, float eps, int zc, uint16_t* y, float* mu, float* rsigma,
                           uint32_t* amax_part, uint8_t* q_row, uint8_t* s_row, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(norm_blocks(rows)), block(kNormThreads);
  const bool am = amax_part != nullptr, mx = q_row != nullptr;
#define SGE_NORM_FWD(L, A, M)                                                                            \
  hipLaunchKernelGGL((norm_fwd_kernel<L, A, M>), grid, block, 0, s, x, gamma, beta, rows, cols, eps, zc, y, mu, \
                     rsigma, amax_part, q_row, s_row)
  if (ln) {
    if (am && mx) SGE_NORM_FWD(true, true, true);
    else if (am) SGE_NORM_FWD(true, true, false);
    else if (mx) SGE_NORM_FWD(true, false, true);
    else SGE_NORM_FWD(true, false, false);
  } else {
    if (am && mx) SGE_NORM_FWD(false, true, true);
    else if (am) SGE_NORM_FWD(false, true, false);
    else if (mx) SGE_NORM_FWD(false, false, true);
    else SGE_NORM_FWD(false, false, false);
  }
#undef SGE_NORM_FWD
  return hipGetLastError();
}

hipError_t launch_norm_bwd(bool ln, const uint16_t* dz, const uint16_t* x, const float* mu, const float* rsigma,
                           const uint16_t* gamma, int64_t rows, int64_t cols, int zc, uint16_t* dx, uint16_t* dgamma,
                           uint16_t* dbeta, float* part, hipStream_t s) {
  const int nb = norm_bwd_blocks(rows);
  float* dg_part = part;
  float* db_part = part + (int64_t)nb * cols;
  if (rows > 0) {
#define SGE_NORM_BWD(L, C)                                                                                      \
  hipLaunchKernelGGL((norm_bwd_kernel<L, C>), dim3(nb), dim3(kNormThreads), 0, s, dz, x, mu, rsigma, gamma, rows, \
                     cols, zc, dx, dg_part, db_part)
    const int64_t nch = (cols / 8 + kNormThreads - 1) / kNormThreads;
    if (nch <= 1) { if (ln) SGE_NORM_BWD(true, 1); else SGE_NORM_BWD(false, 1); }
    else if (nch <= 2) { if (ln) SGE_NORM_BWD(true, 2); else SGE_NORM_BWD(false, 2); }
    else if (nch <= 4) { if (ln) SGE_NORM_BWD(true, 4); else SGE_NORM_BWD(false, 4); }
    else { if (ln) SGE_NORM_BWD(true, 8); else SGE_NORM_BWD(false, 8); }
#undef SGE_NORM_BWD
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    hipError_t e = launch_fill_f32_zero(part, (int64_t)nb * cols * 2, s);   // no rows: zero gradients
    if (e != hipSuccess) return e;
  }
  const dim3 g((unsigned)((cols + 255) / 256));
  hipLaunchKernelGGL(colsum_parts_kernel, g, dim3(256), 0, s, dg_part, nb, cols, dgamma);
  if (ln) hipLaunchKernelGGL(colsum_parts_kernel, g, dim3(256), 0, s, db_part, nb, cols, dbeta);
  return hipGetLastError();
}

}  // namespace sge
