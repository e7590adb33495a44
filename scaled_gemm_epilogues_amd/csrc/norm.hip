// RMSNorm and LayerNorm for gfx950, forward and backward, with the quantized outputs that feed
// a linear ("NVIDIA TransformerEngine PyTorch Ext Normalization", Description and I/O
// Contract: the forward returns the normalized, optionally quantized, output and the saved
// statistics; with current scaling the norm computes its amax and a quantize pass follows;
// MXFP8 is produced by the norm kernel itself; the backward returns dx, dgamma, dbeta).
//
// Forward: one row per block iteration (grid-stride over rows, at most kNormBlocks blocks),
// 256 threads, thread t owning the 8-column chunks 8t + 2048i. Statistics in fp32 with a
// fixed-order block reduction (LayerNorm's variance in a second pass around the mean, over the
// row held in registers; the block's next row is loaded meanwhile); the output is rounded
// once to bf16. With AMAX each block also reduces the bf16 output's
// magnitude into one partial (the current-scaling quantize pass finishes it); with MXROW the
// rowwise MXFP8 copy of the bf16 output is written from registers (four adjacent lanes hold a
// 32-column block), the bytes the standalone quantizer writes for the same bf16 output.
//
// Backward: the same row walk with the row's dz and x held in registers (one HBM read each);
// per row the two means (of d*xhat, and of d for LayerNorm) are block-reduced, dx is written
// in bf16, and each block keeps its own column sums of dz*xhat and dz in registers, stored
// once as fp32 partials; a second kernel adds the partials of all blocks in a fixed order
// (deterministic dgamma / dbeta). Rows stay in registers between passes, and a block loads its
// next row while working the current one.
#include <type_traits>

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

__device__ __forceinline__ float bf16_at(const uint4& u, int e) {
  const uint32_t w = e < 2 ? u.x : (e < 4 ? u.y : (e < 6 ? u.z : u.w));
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// One row's NCH 16-byte chunks per thread (columns 8t + 2048i) as branch-free buffer loads:
// chunks past the row, and every chunk of a row past the end (nbytes 0), read as zeros, so all
// of them are in flight together. A resource per row keeps the offsets 32-bit.
template <int NCH>
__device__ __forceinline__ void load_row(const uint16_t* base, int64_t cols, bool exists, uint4 (&u)[NCH]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, exists ? cols * 2 : 0);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = 8 * (int64_t)threadIdx.x + 2048 * (int64_t)i;
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, c < cols ? (int)(c * 2) : (int)kOOB, 0, 0);
    u[i] = make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
  }
}

template <int NCH>
__device__ __forceinline__ void load_vec(const uint16_t* p, int64_t cols, uint4 (&u)[NCH]) {
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int64_t c = 8 * (int64_t)threadIdx.x + 2048 * (int64_t)i;
    u[i] = c < cols ? *reinterpret_cast<const uint4*>(p + c) : make_uint4(0, 0, 0, 0);
  }
}

// NCH: chunks of 8 columns per thread (cols <= 2048 * NCH). The row stays in registers between
// the statistics and the output, and the block's next row is loaded while this one is worked.
template <bool LN, bool AMAX, bool MXROW, int NCH>
__global__ __launch_bounds__(kNormThreads) void norm_fwd_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma, const uint16_t* __restrict__ beta,
    int64_t rows, int64_t cols, float eps, int zero_centered, uint16_t* __restrict__ y, float* __restrict__ mu_out,
    float* __restrict__ rsigma_out, uint32_t* __restrict__ amax_part, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row) {
  __shared__ float red[kNormThreads / 64];
  const int t = threadIdx.x;
  const float gofs = zero_centered ? 1.0f : 0.0f;
  const float inv_cols = 1.0f / (float)cols;
  uint4 gq[NCH], bq[NCH];
  load_vec<NCH>(gamma, cols, gq);
  if constexpr (LN) load_vec<NCH>(beta, cols, bq);
  uint32_t amax = 0;
  auto work = [&](int64_t r, const uint4 (&ux)[NCH]) {
    float mu = 0.0f;
    if constexpr (LN) {
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) s += bf16_at(ux[i], e);   // zeros past the row
      mu = block_sum_f32(s, red) * inv_cols;
    }
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      if (c < cols) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = bf16_at(ux[i], e) - mu;
          ss += d * d;
        }
      }
    }
    const float rs = 1.0f / sqrtf(block_sum_f32(ss, red) * inv_cols + eps);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      if (c >= cols && !MXROW) continue;
      const bool ok = c < cols;
      v4i vy = {0, 0, 0, 0};
      if (ok) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] = (bf16_at(ux[i], e) - mu) * rs * (bf16_at(gq[i], e) + gofs);
          if constexpr (LN) o[e] += bf16_at(bq[i], e);
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
  };
  const int64_t G = gridDim.x;
  uint4 ua[NCH], ub[NCH];
  int64_t r = blockIdx.x;
  load_row<NCH>(x + r * cols, cols, r < rows, ua);
  for (; r < rows; r += 2 * G) {
    load_row<NCH>(x + (r + G) * cols, cols, r + G < rows, ub);
    work(r, ua);
    if (r + G >= rows) break;
    load_row<NCH>(x + (r + 2 * G) * cols, cols, r + 2 * G < rows, ua);
    work(r + G, ub);
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
  // registers (as loaded bf16) between the reduction pass and the dx pass, and the block's next
  // row (with its statistics) is loaded while this one is worked.
  __shared__ float red[kNormThreads / 64];
  const int t = threadIdx.x;
  const float gofs = zero_centered ? 1.0f : 0.0f;
  const float inv_cols = 1.0f / (float)cols;
  float pg[NCH][8], pb[NCH][8];
  uint4 gq[NCH];
  load_vec<NCH>(gamma, cols, gq);
#pragma unroll
  for (int i = 0; i < NCH; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) pg[i][e] = pb[i][e] = 0.0f;
  struct Row {
    uint4 d[NCH], x[NCH];
    float rs, m;
  };
  auto load = [&](int64_t r, Row& w) {
    const bool ex = r < rows;
    load_row<NCH>(dz + r * cols, cols, ex, w.d);
    load_row<NCH>(x + r * cols, cols, ex, w.x);
    const int64_t rr = ex ? r : 0;                      // a row that exists (rows > 0 here)
    w.rs = rsigma_in[rr];
    w.m = LN ? mu_in[rr] : 0.0f;
  };
  auto work = [&](int64_t r, const Row& w) {
    const float rs = w.rs, m = w.m;
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = bf16_at(w.d[i], e);             // zero past the row
        const float xh = (bf16_at(w.x[i], e) - m) * rs;
        const float dg = d * (bf16_at(gq[i], e) + gofs);
        s1 += dg * xh;
        if constexpr (LN) s2 += dg;
        pg[i][e] += d * xh;
        if constexpr (LN) pb[i][e] += d;
      }
    }
    const float m1 = block_sum_f32(s1, red) * inv_cols;
    const float m2 = LN ? block_sum_f32(s2, red) * inv_cols : 0.0f;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int64_t c = 8 * (int64_t)t + 2048 * (int64_t)i;
      if (c < cols) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (bf16_at(w.x[i], e) - m) * rs;
          o[e] = rs * (bf16_at(w.d[i], e) * (bf16_at(gq[i], e) + gofs) - m2 - xh * m1);
        }
        *reinterpret_cast<v4i*>(dx + r * cols + c) =
            v4i{(int)pack_bf16x2(o[0], o[1]), (int)pack_bf16x2(o[2], o[3]), (int)pack_bf16x2(o[4], o[5]),
                (int)pack_bf16x2(o[6], o[7])};
      }
    }
  };
  const int64_t G = gridDim.x;
  Row ra, rb;
  int64_t r = blockIdx.x;
  load(r, ra);
  for (; r < rows; r += 2 * G) {
    load(r + G, rb);
    work(r, ra);
    if (r + G >= rows) break;
    load(r + 2 * G, ra);
    work(r + G, rb);
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

// out[c] = bf16 of the sum over parts b of part[b][c] in a fixed order: eight groups of threads
// per column each add the parts b = g, g + 8, g + 16, ... in turn (loads in flight together),
// then the eight group sums are added in group order.
constexpr int kCsCols = 32, kCsGroups = 8;
__global__ __launch_bounds__(kCsCols * kCsGroups) void colsum_parts_kernel(const float* __restrict__ part, int nparts,
                                                                         int64_t cols, uint16_t* __restrict__ out) {
  __shared__ float red[kCsGroups][kCsCols];
  const int tx = threadIdx.x % kCsCols, ty = threadIdx.x / kCsCols;
  const int64_t c = (int64_t)blockIdx.x * kCsCols + tx;
  float s = 0.0f;
  if (c < cols) {
#pragma unroll 8
    for (int b = ty; b < nparts; b += kCsGroups) s += part[(int64_t)b * cols + c];
  }
  red[ty][tx] = s;
  __syncthreads();
  if (ty == 0 && c < cols) {
    float t = red[0][tx];
#pragma unroll
    for (int g = 1; g < kCsGroups; ++g) t += red[g][tx];
    out[c] = f32_to_bf16(t);
  }
}

int norm_blocks(int64_t rows) { return (int)(rows < kNormBlocks ? (rows < 1 ? 1 : rows) : kNormBlocks); }
int norm_bwd_blocks(int64_t rows) { return (int)(rows < kNormBwdBlocks ? (rows < 1 ? 1 : rows) : kNormBwdBlocks); }

hipError_t launch_norm_fwd(bool ln, const uint16_t* x, const uint16_t* gamma, const uint16_t* beta, int64_t rows,
                           int64_t cols, float eps, int zc, uint16_t* y, float* mu, float* rsigma,
                           uint32_t* amax_part, uint8_t* q_row, uint8_t* s_row, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const dim3 grid(norm_blocks(rows)), block(kNormThreads);
  const bool am = amax_part != nullptr, mx = q_row != nullptr;
  const int64_t nch = (cols / 8 + kNormThreads - 1) / kNormThreads;
  auto go = [&](auto lnc, auto amc, auto mxc) {
    constexpr bool L = decltype(lnc)::value, A = decltype(amc)::value, M = decltype(mxc)::value;
#define SGE_NORM_FWD(C)                                                                                          \
  hipLaunchKernelGGL((norm_fwd_kernel<L, A, M, C>), grid, block, 0, s, x, gamma, beta, rows, cols, eps, zc, y, mu, \
                     rsigma, amax_part, q_row, s_row)
    if (nch <= 1) SGE_NORM_FWD(1);
    else if (nch <= 2) SGE_NORM_FWD(2);
    else if (nch <= 4) SGE_NORM_FWD(4);
    else SGE_NORM_FWD(8);
#undef SGE_NORM_FWD
  };
  using T = std::true_type;
  using F = std::false_type;
  if (ln) {
    if (am && mx) go(T{}, T{}, T{});
    else if (am) go(T{}, T{}, F{});
    else if (mx) go(T{}, F{}, T{});
    else go(T{}, F{}, F{});
  } else {
    if (am && mx) go(F{}, T{}, T{});
    else if (am) go(F{}, T{}, F{});
    else if (mx) go(F{}, F{}, T{});
    else go(F{}, F{}, F{});
  }
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
  const dim3 g((unsigned)((cols + kCsCols - 1) / kCsCols));
  hipLaunchKernelGGL(colsum_parts_kernel, g, dim3(kCsCols * kCsGroups), 0, s, dg_part, nb, cols, dgamma);
  if (ln) hipLaunchKernelGGL(colsum_parts_kernel, g, dim3(kCsCols * kCsGroups), 0, s, db_part, nb, cols, dbeta);
  return hipGetLastError();
}

}  // namespace sge
