// Small kernels of the grouped path: split offsets, the unfused scaled SwiGLU,
// the deterministic reduction of per-tile dprobs partials, and zero fills.
#include "common.h"
#include "launch.h"

namespace sge {

// ------------------------------------------------------------ zero fills
__global__ void fill_bf16_zero_kernel(uint16_t* c, int64_t rows, int64_t cols, int64_t ld) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    c[(i / cols) * ld + i % cols] = 0;
}

hipError_t launch_fill_bf16_zero(uint16_t* c, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  const int64_t n = rows * cols;
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_bf16_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s,
                     c, rows, cols, ld);
  return hipGetLastError();
}

__global__ void fill_f32_zero_kernel(float* c, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    c[i] = 0.0f;
}

hipError_t launch_fill_f32_zero(float* c, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fill_f32_zero_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, c,
                     n);
  return hipGetLastError();
}

// -------------------------------------------------------- split offsets
// "Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
// (Description, Precomputed Tensor Offsets Optimization): offsets computed once
// on the device from the split sizes and reused by forward and backward.
struct Mults {
  int64_t v[8];
};

constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kScanThreads) void splits_to_offsets_kernel(const int64_t* __restrict__ splits,
                                                                         int G, Mults mults, int n_mult,
                                                                         int64_t expected_total,
                                                                         int64_t* __restrict__ offsets,
                                                                         int32_t* err_flag) {
  __shared__ int64_t part[kScanThreads];
  __shared__ int bad_shared;
  const int t = threadIdx.x;
  if (t == 0) bad_shared = 0;
  // Each thread owns a contiguous run of groups.
  const int per = (G + kScanThreads - 1) / kScanThreads;
  const int g0 = t * per;
  const int g1 = g0 + per < G ? g0 + per : G;
  int64_t local = 0;
  int bad = 0;
  for (int g = g0; g < g1; ++g) {
    const int64_t s = splits[g];
    bad |= s < 0;
    local += s;
  }
  part[t] = local;
  __syncthreads();
  if (bad) atomicOr(&bad_shared, 1);
  // Inclusive Hillis-Steele scan over the per-thread sums.
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int64_t add = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int64_t run = t > 0 ? part[t - 1] : 0;   // exclusive prefix of this thread's run
  for (int g = g0; g < g1; ++g) {
    for (int i = 0; i < n_mult; ++i) offsets[(int64_t)i * (G + 1) + g] = run * mults.v[i];
    run += splits[g];
  }
  if (t == kScanThreads - 1) {
    const int64_t total = part[kScanThreads - 1];
    for (int i = 0; i < n_mult; ++i) offsets[(int64_t)i * (G + 1) + G] = total * mults.v[i];
  }
  __syncthreads();
  if (t == kScanThreads - 1 && err_flag) {
    const int64_t total = part[kScanThreads - 1];
    *err_flag = (bad_shared || (expected_total >= 0 && total != expected_total)) ? 1 : 0;
  }
}

hipError_t launch_splits_to_offsets(const int64_t* splits, int G, const int64_t* mults, int n_mult,
                                    int64_t expected_total, int64_t* offsets, int32_t* err_flag,
                                    hipStream_t s) {
  Mults m{};
  for (int i = 0; i < n_mult; ++i) m.v[i] = mults[i];
  hipLaunchKernelGGL(splits_to_offsets_kernel, dim3(1), dim3(kScanThreads), 0, s, splits, G, m, n_mult,
                     expected_total, offsets, err_flag);
  return hipGetLastError();
}

// ------------------------------------- token-blocked MXFP8 group layout
// Operands of a grouped wgrad are quantized in blocks of 32 along the tokens of each group,
// each group stored from a position aligned to `align` tokens. One block computes
//   c[g]   = the offsets as every grouped call reads them (clamped into [0, T], non-decreasing)
//   pad[g] = pad[g-1] + roundup(c[g] - c[g-1], align), pad[0] = 0
// into layout[0][..] and layout[1][..] ([2][G+1] int64), G + 1 <= kLayoutMax.
constexpr int kLayoutMax = 4097;

__global__ __launch_bounds__(kScanThreads) void mx_group_layout_kernel(const int64_t* __restrict__ offsets, int G,
                                                                       int64_t T, int64_t align,
                                                                       int64_t* __restrict__ layout) {
  __shared__ int64_t part[kScanThreads];
  __shared__ int64_t cs[kLayoutMax];
  const int t = threadIdx.x;
  const int n = G + 1;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int i0 = t * per, i1 = i0 + per < n ? i0 + per : n;
  // clamped offsets: running max of min(offsets[i], T), from 0
  int64_t m = 0;
  for (int i = i0; i < i1; ++i) {
    const int64_t v = offsets[i] < T ? offsets[i] : T;
    m = v > m ? v : m;
  }
  part[t] = m;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int64_t other = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] = other > part[t] ? other : part[t];
    __syncthreads();
  }
  int64_t run = t > 0 ? part[t - 1] : 0;
  for (int i = i0; i < i1; ++i) {
    const int64_t v = offsets[i] < T ? offsets[i] : T;
    run = v > run ? v : run;
    cs[i] = run;
    layout[i] = run;
  }
  __syncthreads();
  // aligned starts: exclusive prefix sum of the rounded-up group lengths
  int64_t sum = 0;
  for (int g = i0; g < i1 && g < G; ++g) sum += (cs[g + 1] - cs[g] + align - 1) / align * align;
  part[t] = sum;
  __syncthreads();
  for (int o = 1; o < kScanThreads; o <<= 1) {
    const int64_t add = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int64_t pos = t > 0 ? part[t - 1] : 0;
  for (int g = i0; g < i1 && g < G; ++g) {
    layout[n + g] = pos;
    pos += (cs[g + 1] - cs[g] + align - 1) / align * align;
  }
  if (t == kScanThreads - 1) layout[n + G] = part[kScanThreads - 1];
}

hipError_t launch_mx_group_layout(const int64_t* offsets, int G, int64_t T, int64_t align, int64_t* layout,
                                  hipStream_t s) {
  if (G + 1 > kLayoutMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mx_group_layout_kernel, dim3(1), dim3(kScanThreads), 0, s, offsets, G, T, align, layout);
  return hipGetLastError();
}

// ------------------------------------------------ unfused scaled SwiGLU
__device__ __forceinline__ float sigmoid_f(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// One block per token row; 8 columns per thread per step.
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t* __restrict__ h,
                                                        const float* __restrict__ p, uint16_t* __restrict__ y,
                                                        int64_t F) {
  const int64_t t = blockIdx.x;
  const float pt = p[t];
  const uint16_t* hr = h + t * 2 * F;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < F; c += 256 * 8) {
    const uint4 av = *reinterpret_cast<const uint4*>(hr + c);
    const uint4 bv = *reinterpret_cast<const uint4*>(hr + F + c);
    const uint32_t aw[4] = {av.x, av.y, av.z, av.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a0 = bf16_lo(aw[e]), a1 = bf16_hi(aw[e]), b0 = bf16_lo(bw[e]), b1 = bf16_hi(bw[e]);
      o[e] = pack_bf16x2(pt * (a0 * sigmoid_f(a0)) * b0, pt * (a1 * sigmoid_f(a1)) * b1);
    }
    *reinterpret_cast<uint4*>(y + t * F + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

hipError_t launch_swiglu_fwd(const uint16_t* h, const float* p, uint16_t* y, int64_t T, int64_t F, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3((unsigned)T), dim3(256), 0, s, h, p, y, F);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t* __restrict__ gy,
                                                        const uint16_t* __restrict__ h,
                                                        const float* __restrict__ p, uint16_t* __restrict__ dh,
                                                        float* __restrict__ dp, int64_t F) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const float pt = p[t];
  const uint16_t* hr = h + t * 2 * F;
  float part = 0.0f;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < F; c += 256 * 8) {
    const uint4 gv = *reinterpret_cast<const uint4*>(gy + t * F + c);
    const uint4 av = *reinterpret_cast<const uint4*>(hr + c);
    const uint4 bv = *reinterpret_cast<const uint4*>(hr + F + c);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, aw[4] = {av.x, av.y, av.z, av.w},
                   bw[4] = {bv.x, bv.y, bv.z, bv.w};
    uint32_t da[4], db[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float dav[2], dbv[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float g = k ? bf16_hi(gw[e]) : bf16_lo(gw[e]);
        const float a = k ? bf16_hi(aw[e]) : bf16_lo(aw[e]);
        const float b = k ? bf16_hi(bw[e]) : bf16_lo(bw[e]);
        const float sg = sigmoid_f(a);
        const float silu = a * sg;
        dav[k] = g * pt * b * (sg * (1.0f + a * (1.0f - sg)));
        dbv[k] = g * pt * silu;
        part += g * silu * b;
      }
      da[e] = pack_bf16x2(dav[0], dav[1]);
      db[e] = pack_bf16x2(dbv[0], dbv[1]);
    }
    *reinterpret_cast<uint4*>(dh + t * 2 * F + c) = make_uint4(da[0], da[1], da[2], da[3]);
    *reinterpret_cast<uint4*>(dh + t * 2 * F + F + c) = make_uint4(db[0], db[1], db[2], db[3]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) dp[t] = (red[0] + red[1]) + (red[2] + red[3]);
}

hipError_t launch_swiglu_bwd(const uint16_t* gy, const uint16_t* h, const float* p, uint16_t* dh, float* dp,
                             int64_t T, int64_t F, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3((unsigned)T), dim3(256), 0, s, gy, h, p, dh, dp, F);
  return hipGetLastError();
}

// ------------------------------------- deterministic dprobs reduction
// out[t] = sum over parts (fixed order) for tokens inside the groups, 0 elsewhere.
__global__ void rowsum_parts_kernel(const float* __restrict__ part, int nparts, const int64_t* __restrict__ offsets,
                                    int G, int64_t T, float* __restrict__ out) {
  int64_t lo = offsets[0], hi = offsets[G];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T; t += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    if (t >= lo && t < hi) {
      for (int i = 0; i < nparts; ++i) s += part[(int64_t)i * T + t];
    }
    out[t] = s;
  }
}

hipError_t launch_rowsum_parts(const float* part, int nparts, const int64_t* offsets, int G, int64_t T, float* out,
                               hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const int64_t blocks = (T + 255) / 256;
  hipLaunchKernelGGL(rowsum_parts_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, s, part,
                     nparts, offsets, G, T, out);
  return hipGetLastError();
}

}  // namespace sge
