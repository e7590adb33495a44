// Quantizers for gfx950: FP8 E4M3 with per-tensor current scaling, and MXFP8.
//
// Current scaling is "amax, then quantize" ("NVIDIA TransformerEngine PyTorch
// Ext Normalization", Description): an HBM pass reduces max|x| block-wise, a
// second pass finishes the reduction in every block (a few KB from L2), derives
// scale = 448/amax and writes the E4M3 bytes (and optionally their transpose,
// the operand layout the backward GEMMs read).
//
// MXFP8 ("core.tensor_parallel.inference_layers", _apply_linear with an MXFP8
// weight) uses one E8M0 exponent per 32 elements: X = floor(log2(amax)) - 8
// (OCP MX v1.0 section 6.3), clamped to [-127, 127]. One pass reads each bf16
// element once and writes both the rowwise and the columnwise (transposed)
// copy. The per-block amax is an integer max over bf16 bit patterns with the
// sign cleared, which orders like the magnitudes.
#include <mutex>

#include "common.h"
#include "launch.h"

namespace sge {

constexpr int kAmaxThreads = 256;

__device__ __forceinline__ uint32_t absmax_bits2(uint32_t d) {
  const uint32_t lo = d & 0x7FFFu, hi = (d >> 16) & 0x7FFFu;
  return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t absmax_bits8(const uint4& v) {
  uint32_t a = absmax_bits2(v.x), b = absmax_bits2(v.y), c = absmax_bits2(v.z), d = absmax_bits2(v.w);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Block-wide max of one uint32 per thread (all threads must call).
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t m = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) m = red[w] > m ? red[w] : m;
  __syncthreads();
  return m;
}

__global__ __launch_bounds__(kAmaxThreads) void amax_partial_kernel(const uint16_t* __restrict__ src,
                                                                    int64_t n, uint32_t* __restrict__ partial) {
  __shared__ uint32_t red[kAmaxThreads / 64];
  const int64_t nvec = n >> 3;
  const int64_t stride = (int64_t)gridDim.x * kAmaxThreads;
  const uint4* v = reinterpret_cast<const uint4*>(src);
  uint32_t m = 0;
  int64_t i = (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const uint4 a = v[i], b = v[i + stride], c = v[i + 2 * stride], d = v[i + 3 * stride];
    uint32_t x = absmax_bits8(a), y = absmax_bits8(b), z = absmax_bits8(c), w = absmax_bits8(d);
    x = x > y ? x : y;
    z = z > w ? z : w;
    x = x > z ? x : z;
    m = m > x ? m : x;
  }
  for (; i < nvec; i += stride) {
    const uint32_t x = absmax_bits8(v[i]);
    m = m > x ? m : x;
  }
  for (int64_t t = nvec * 8 + (int64_t)blockIdx.x * kAmaxThreads + threadIdx.x; t < n; t += stride) {
    const uint32_t x = src[t] & 0x7FFFu;
    m = m > x ? m : x;
  }
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = m;
}

// The 16-byte chunks at column c of rows lr0 + 32k (k = 0..3) of a 128-row tile whose first row
// is r0 and which has nrows rows (rows past them, and columns past cols, read as zeros): branch-
// free buffer loads, so all four are in flight together. Offsets fit in 31 bits (the callers
// refuse rows longer than 2^22 elements).
__device__ __forceinline__ void load_rows4(const uint16_t* src, int64_t r0, int64_t nrows, int64_t cols, int64_t c,
                                          int lr0, uint4 (&v)[4]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + r0 * cols, (nrows < 128 ? nrows : 128) * cols * 2);
  const uint32_t cb = c < cols ? (uint32_t)(c * 2) : kOOB;
  const uint32_t rb = (uint32_t)(cols * 2);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(cb + (uint32_t)(lr0 + 32 * k) * rb), 0, 0);
    v[k] = make_uint4((uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]);
  }
}

int amax_partial_blocks(int64_t n) {
  const int64_t want = (n / 8 + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
  return (int)(want < 1 ? 1 : (want > 1024 ? 1024 : want));
}

// Partials of the per-tensor amax for callers that cannot allocate (the no-allocation variant of
// the FP8 current-scaling quantizer): one array per GPU, held until the process ends, as large as
// the most partials amax_partial_blocks() asks for. Host code never passes the array's name to a
// kernel (on the host it only stands for the symbol); it takes the device address that
// hipGetSymbolAddress returns for the current device, looked up once per device.
constexpr int kScratchPartials = 1024;
static __device__ __align__(256) uint32_t scratch[kScratchPartials];

hipError_t amax_scratch(uint32_t** partial, size_t* bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static uint32_t* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<uint32_t*>(p);
  }
  *partial = addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_amax_partial(const uint16_t* src, int64_t n, uint32_t* partial, int nblocks,
                               hipStream_t s) {
  hipLaunchKernelGGL(amax_partial_kernel, dim3(nblocks), dim3(kAmaxThreads), 0, s, src, n, partial);
  return hipGetLastError();
}

// Current scaling from an amax: scale = 448 / amax (IEEE division, no fast-math; 1 for an
// all-zero tensor; clamped to the largest finite fp32), scale_inv = 1 / scale.
__device__ __forceinline__ void fp8_scales(float amax, float& scale, float& scale_inv) {
  scale = 1.0f;
  if (amax > 0.0f) {
    scale = 448.0f / amax;
    if (scale > 3.402823466e38f) scale = 3.402823466e38f;
  }
  scale_inv = 1.0f / scale;
}

// Tiles of a grouped tensor walk the stored positions of a group layout ([2][G+1]: token
// ranges c[], aligned starts pad[]): a tile of 128 positions lies inside one group's aligned
// range. Returns false past the last group; else the group, the tile's first source row and
// how many of its rows exist (the rest of the 128 positions are padding). With no layout the
// G groups are equal runs of rows / G rows (a multiple of 128) and positions are rows.
__device__ __forceinline__ bool group_tile(const int64_t* __restrict__ layout, int G, int64_t rows, int64_t p0,
                                           int& g, int64_t& r0, int64_t& nrows) {
  if (!layout) {
    if (p0 >= rows) return false;
    const int64_t per = rows / G;
    g = (int)(p0 / per);
    r0 = p0;
    nrows = (int64_t)(g + 1) * per - p0;
    return true;
  }
  const int64_t* c = layout;
  const int64_t* pad = layout + G + 1;
  if (p0 >= pad[G]) return false;
  int lo = 0, hi = G - 1;                               // last g with pad[g] <= p0
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pad[mid] <= p0) lo = mid;
    else hi = mid - 1;
  }
  g = lo;
  r0 = c[lo] + (p0 - pad[lo]);
  nrows = c[lo + 1] - r0;                               // >= 1: aligned lengths round up
  // a layout not made for these rows reads nothing out of range
  r0 = r0 < 0 ? 0 : (r0 > rows ? rows : r0);
  nrows = nrows > rows - r0 ? rows - r0 : nrows;
  return true;
}

// The dispatcher hands workgroups to the 8 XCDs round-robin (workgroup b runs on XCD b % 8),
// each with its own L2. Renumbering tiles so that XCD x takes one contiguous range makes the
// tiles an XCD runs together neighbours (a tile's 64-byte rowwise output rows are half a
// 128-byte line whose other half the next column tile writes). Bijective on [0, total).
// Used by the grouped quantizers, where it measured 3-13% faster.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t total) {
  const int64_t x = bid & 7, i = bid >> 3;
  const int64_t q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + i;
}

// Tiles of 128 rows x 64 columns; 256 threads, 8 bf16 (16 B) per thread per pass. The
// transposed copy is written through LDS so each column's 128 rows leave as one 128-byte
// line. Tiles are visited in the reverse order of the amax pass, which left the most
// recently read part of the tensor in the last-level cache.
constexpr int kQR = 128, kQC = 64;

__global__ __launch_bounds__(256) void quantize_fp8_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols, const uint32_t* __restrict__ partial,
    int nparts, uint8_t* __restrict__ q, uint8_t* __restrict__ q_t, float* amax_out, float* scale_out,
    float* scale_inv_out) {
  __shared__ uint32_t red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQC][kQR + 16];   // [column][row]

  // Finish the amax: every block reduces the partials itself (no grid barrier).
  uint32_t m = 0;
  for (int i = threadIdx.x; i < nparts; i += blockDim.x) m = partial[i] > m ? partial[i] : m;
  m = block_max_u32(m, red);
  const float amax = __builtin_bit_cast(float, m << 16);
  float scale, scale_inv;
  fp8_scales(amax, scale, scale_inv);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    *amax_out = amax;
    *scale_out = scale;
    *scale_inv_out = scale_inv;
  }

  const int64_t tr = (rows + kQR - 1) / kQR;
  const int64_t tc = (cols + kQC - 1) / kQC;
  const int64_t ntiles = tr * tc;
  const int t = threadIdx.x;
  const int cchunk = t & 7;          // 8 columns each
  const int rsub = t >> 3;           // 0..31
  for (int64_t it = blockIdx.x; it < ntiles; it += gridDim.x) {
    const int64_t tile_id = ntiles - 1 - it;
    const int64_t r0 = (tile_id / tc) * kQR, c0 = (tile_id % tc) * kQC;
    uint4 vv[4];
    load_rows4(src, r0, rows - r0, cols, c0 + cchunk * 8, rsub, vv);
#pragma unroll
    for (int pass = 0; pass < kQR / 32; ++pass) {
      const int lr = rsub + 32 * pass;
      const int64_t r = r0 + lr, c = c0 + cchunk * 8;
      uint32_t b[4] = {0, 0, 0, 0};
      if (r < rows && c < cols) {
        const uint4 v = vv[pass];
        b[0] = e4m3x2(bf16_lo(v.x) * scale, bf16_hi(v.x) * scale);
        b[1] = e4m3x2(bf16_lo(v.y) * scale, bf16_hi(v.y) * scale);
        b[2] = e4m3x2(bf16_lo(v.z) * scale, bf16_hi(v.z) * scale);
        b[3] = e4m3x2(bf16_lo(v.w) * scale, bf16_hi(v.w) * scale);
        if (q) *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
      }
      if (q_t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          tile[cchunk * 8 + 2 * e][lr] = (uint8_t)(b[e] & 0xFF);
          tile[cchunk * 8 + 2 * e + 1][lr] = (uint8_t)(b[e] >> 8);
        }
      }
    }
    if (q_t) {
      __syncthreads();
      // Thread -> one column, 32 consecutive rows (2 x 16 bytes) of the transposed output.
      const int lc = t >> 2, seg = (t & 3) * 32;
      const int64_t c = c0 + lc, r = r0 + seg;
      if (c < cols && r < rows) {
        const uint4 lo = *reinterpret_cast<const uint4*>(&tile[lc][seg]);
        const uint4 hi = *reinterpret_cast<const uint4*>(&tile[lc][seg + 16]);
        *reinterpret_cast<uint4*>(q_t + c * rows + r) = lo;
        if (r + 16 < rows) *reinterpret_cast<uint4*>(q_t + c * rows + r + 16) = hi;
      }
      __syncthreads();
    }
  }
}

hipError_t launch_quantize_fp8(const uint16_t* src, int64_t rows, int64_t cols, const uint32_t* partial,
                               int nparts, uint8_t* q, uint8_t* q_t, float* amax, float* scale,
                               float* scale_inv, hipStream_t s) {
  const int64_t tiles = ((rows + kQR - 1) / kQR) * ((cols + kQC - 1) / kQC);
  const int grid = (int)(tiles < 2048 ? (tiles < 1 ? 1 : tiles) : 2048);
  hipLaunchKernelGGL(quantize_fp8_kernel, dim3(grid), dim3(256), 0, s, src, rows, cols, partial, nparts, q,
                     q_t, amax, scale, scale_inv);
  return hipGetLastError();
}


// MX tile: 128 rows x C columns (C = 128 dense, 64 token-blocked); 4C threads; thread t owns
// columns 8*(t%(C/8))..+7 of rows t/(C/8) + 32k, k = 0..3. Rowwise blocks are 4 consecutive
// threads of a row; columnwise blocks are the 32 rows of one k, reduced across lanes and
// waves. The columnwise copy goes through LDS so each column's 128 rows leave as one 128-byte
// line (and with C = 128 each row's rowwise codes do too).
//
// GROUPED: the columnwise copy is blocked along the tokens of each group. Tiles then walk the
// stored (aligned) token positions: a tile of 128 positions lies inside one group's aligned
// range, reads that group's tokens (zeros past its end) and writes all 128 positions, so the
// padding between groups comes out as zero codes under all-zero blocks (E8M0 byte 0).
// Tile width: 128 columns when the rowwise copy is written in the dense layout (8-10% faster
// than 64 on a 16384 x 8192 tensor: each row's codes leave as one 128-byte line), 64 for the
// token-blocked layout and for the columnwise copy alone (4-22% and 9% faster there).
constexpr int kMR = 128;
template <bool WIDE>
struct MxTile {
  static constexpr int kC = WIDE ? 128 : 64;           // columns
  static constexpr int kThreads = 32 * (kC / 8);       // each thread: 8 columns of 4 rows (32 apart)
};

template <bool GROUPED, bool WIDE>
__global__ __launch_bounds__(MxTile<WIDE>::kThreads) void quantize_mxfp8_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols, uint8_t* __restrict__ q_row,
    uint8_t* __restrict__ s_row, uint8_t* __restrict__ q_colT, uint8_t* __restrict__ s_colT, int G,
    const int64_t* __restrict__ layout, int64_t ld_t) {
  constexpr int kMC = MxTile<WIDE>::kC;
  __shared__ __attribute__((aligned(16))) uint16_t xt[kMC][kMR + 8];    // [column][row] bf16 bits
  const int64_t tc = (cols + kMC - 1) / kMC;
  // Grouped (token-blocked) tiles in XCD-contiguous ranges: measured 5% faster there, while
  // the dense order suits the dense layout better (7-10% faster on a 16384 x 8192 tensor).
  const int64_t tile = GROUPED ? xcd_tile(blockIdx.x, gridDim.x) : (int64_t)blockIdx.x;
  const int64_t p0 = (tile / tc) * kMR;                   // first row (dense) or stored position
  const int64_t c0 = (tile % tc) * kMC;
  int64_t r0 = p0;               // first source row of the tile
  int64_t nrows = rows - p0;     // source rows of the tile that exist
  int64_t npos = rows - p0;      // columnwise positions the tile writes
  if constexpr (GROUPED) {
    int g;
    if (!group_tile(layout, G, rows, p0, g, r0, nrows)) return;   // past the last group (block-uniform)
    npos = kMR;                                           // pad[g + 1] - p0 >= 128
  }
  const int t = threadIdx.x;
  const int lr = t / (kMC / 8);          // 0..31
  const int cc = t % (kMC / 8);          // column chunk of 8
  const int64_t c = c0 + cc * 8;
  bool ok[4];
  uint4 vv[4];
  load_rows4(src, r0, nrows, cols, c, lr, vv);
#pragma unroll
  for (int k = 0; k < 4; ++k) ok[k] = lr + 32 * k < nrows && c < cols;

  if (q_row) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // Rowwise: a 32-column block is 4 consecutive threads of one row (every lane takes part).
      int e8;
      const v2i qv = mx_quant_lane8(v4i{(int)vv[k].x, (int)vv[k].y, (int)vv[k].z, (int)vv[k].w}, e8);
      if (ok[k]) {
        const int64_t r = r0 + lr + 32 * k;
        *reinterpret_cast<v2i*>(q_row + r * cols + c) = qv;
        if ((cc & 3) == 0) s_row[r * (cols / 32) + (c >> 5)] = (uint8_t)e8;
      }
    }
  }

  if (q_colT) {
    // Columnwise: the tile goes to LDS transposed ([column][row] bf16), then thread t owns
    // the block of rows 32k..32k+31 (k = t % 4) of column t / 4: local amax, 32 codes,
    // written as 32 contiguous bytes (each column's 128 rows leave as one line).
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w[4] = {vv[k].x, vv[k].y, vv[k].z, vv[k].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) xt[cc * 8 + e][lr + 32 * k] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
    __syncthreads();
    const int col = t >> 2, k = t & 3;
    const uint4* seg = reinterpret_cast<const uint4*>(&xt[col][32 * k]);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = seg[i];
      w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
    }
    uint32_t m2 = 0;                                     // rows of one column, two per word
#pragma unroll
    for (int i = 0; i < 16; ++i) m2 = pk_absmax_bits(m2, w[i]);
    const int X = mx_exponent((m2 & 0xFFFFu) > (m2 >> 16) ? (m2 & 0xFFFFu) : (m2 >> 16));
    const uint32_t bound = mx_bound_bits(X) * 0x10001u;
    const float sc = mx_scale_operand(X);
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = e4m3x4_scaled(clamp_pair(w[2 * i], bound), clamp_pair(w[2 * i + 1], bound), sc);
    const int64_t ldc = GROUPED ? ld_t : rows;
    if (c0 + col < cols && 32 * k < npos) {
      uint8_t* dst = q_colT + (c0 + col) * ldc + p0 + 32 * k;
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
      s_colT[(c0 + col) * (ldc / 32) + (p0 >> 5) + k] = (uint8_t)(X + 127);
    }
  }
}

hipError_t launch_quantize_mxfp8(const uint16_t* src, int64_t rows, int64_t cols, uint8_t* q_row,
                                 uint8_t* s_row, uint8_t* q_colT, uint8_t* s_colT, hipStream_t s) {
  if (!q_row) {                                          // the columnwise copy alone
    constexpr int kMC = MxTile<false>::kC;
    const int64_t tiles = ((rows + kMR - 1) / kMR) * ((cols + kMC - 1) / kMC);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL((quantize_mxfp8_kernel<false, false>), dim3((unsigned)tiles), dim3(MxTile<false>::kThreads),
                       0, s, src, rows, cols, q_row, s_row, q_colT, s_colT, 0, nullptr, (int64_t)0);
    return hipGetLastError();
  }
  constexpr int kMC = MxTile<true>::kC;
  const int64_t tiles = ((rows + kMR - 1) / kMR) * ((cols + kMC - 1) / kMC);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((quantize_mxfp8_kernel<false, true>), dim3((unsigned)tiles), dim3(MxTile<true>::kThreads), 0, s,
                     src, rows, cols, q_row, s_row, q_colT, s_colT, 0, nullptr, (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_grouped(const uint16_t* src, int64_t rows, int64_t cols, int G,
                                         const int64_t* layout, int64_t ld_t, uint8_t* q_row, uint8_t* s_row,
                                         uint8_t* q_colT, uint8_t* s_colT, hipStream_t s) {
  // one tile per 128 stored positions (ld_t bounds every group's aligned end) x kMC columns
  constexpr int kMC = MxTile<false>::kC;
  const int64_t tiles = (ld_t / kMR) * ((cols + kMC - 1) / kMC);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((quantize_mxfp8_kernel<true, false>), dim3((unsigned)tiles), dim3(MxTile<false>::kThreads), 0, s,
                     src, rows, cols, q_row, s_row, q_colT, s_colT, G, layout, ld_t);
  return hipGetLastError();
}

// ------------------------------------------- FP8 current scaling per group
// One amax and scale per group (a group quantize with one quantizer per group). Pass 1: each
// block takes 128 stored positions x 512 columns of one group and folds its amax into the
// group's slot with an atomic max over bf16 magnitude bits (order-free, so deterministic).
// Pass 2 quantizes tiles of 128 positions x 64 columns with their group's scale, writing the
// rowwise bytes and the transposed copy (all 128 positions: padding comes out as zero codes).
constexpr int kGAC = 512;

__global__ __launch_bounds__(256) void amax_grouped_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                          int64_t cols, int G, const int64_t* __restrict__ layout,
                                                          float* __restrict__ amax_g) {
  __shared__ uint32_t red[4];
  const int64_t tc = (cols + kGAC - 1) / kGAC;
  const int64_t p0 = (int64_t)(blockIdx.x / tc) * kQR;
  const int64_t c0 = (int64_t)(blockIdx.x % tc) * kGAC;
  int g;
  int64_t r0, nrows;
  if (!group_tile(layout, G, rows, p0, g, r0, nrows)) return;   // block-uniform
  const int t = threadIdx.x;
  const int64_t c = c0 + (t & 63) * 8;
  // Branch-free buffer loads over the tile's existing rows (the rest, and columns past the end,
  // read as zeros, which leave a magnitude maximum unchanged), so a thread's loads are all in
  // flight together. Offsets fit in 31 bits: 128 rows of a row at most 2^22 bf16 long.
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + r0 * cols, (nrows < kQR ? nrows : kQR) * cols * 2);
  const uint32_t cb = c < cols ? (uint32_t)(c * 2) : kOOB;
  const uint32_t rb = (uint32_t)(cols * 2);
  uint32_t m = 0;
#pragma unroll 8
  for (int lr = t >> 6; lr < kQR; lr += 4) {
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(cb + (uint32_t)lr * rb), 0, 0);
    const uint32_t x = absmax_bits8(make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]));
    m = m > x ? m : x;
  }
  m = block_max_u32(m, red);
  // non-negative floats order like their bit patterns: an integer max of (bf16 bits << 16)
  if (t == 0 && m) atomicMax(reinterpret_cast<uint32_t*>(amax_g) + g, m << 16);
}

__global__ __launch_bounds__(256) void quantize_fp8_grouped_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols, int G, const int64_t* __restrict__ layout,
    int64_t ld_t, const float* __restrict__ amax_g, uint8_t* __restrict__ q, uint8_t* __restrict__ q_t,
    float* amax_out, float* scale_out, float* scale_inv_out) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kQC][kQR + 16];   // [column][position]
  const int t = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int gg = t; gg < G; gg += blockDim.x) {
      const float a = amax_g[gg];
      float sc, si;
      fp8_scales(a, sc, si);
      amax_out[gg] = a;
      scale_out[gg] = sc;
      scale_inv_out[gg] = si;
    }
  }
  const int64_t tc = (cols + kQC - 1) / kQC;
  // XCD-contiguous ranges, each walked from its end: the amax pass went the other way, so the
  // tiles it read last (still in the last-level cache) come first
  const int64_t tid = gridDim.x - 1 - xcd_tile(blockIdx.x, gridDim.x);
  const int64_t p0 = (tid / tc) * kQR;
  const int64_t c0 = (tid % tc) * kQC;
  int g;
  int64_t r0, nrows;
  if (!group_tile(layout, G, rows, p0, g, r0, nrows)) return;   // block-uniform
  float scale, scale_inv;
  fp8_scales(amax_g[g], scale, scale_inv);
  const int cchunk = t & 7;
  const int rsub = t >> 3;
  uint4 vv[4];
  load_rows4(src, r0, nrows, cols, c0 + cchunk * 8, rsub, vv);
#pragma unroll
  for (int pass = 0; pass < kQR / 32; ++pass) {
    const int lr = rsub + 32 * pass;
    const int64_t r = r0 + lr, c = c0 + cchunk * 8;
    uint32_t b[4] = {0, 0, 0, 0};
    if (lr < nrows && c < cols) {
      const uint4 v = vv[pass];
      b[0] = e4m3x2(bf16_lo(v.x) * scale, bf16_hi(v.x) * scale);
      b[1] = e4m3x2(bf16_lo(v.y) * scale, bf16_hi(v.y) * scale);
      b[2] = e4m3x2(bf16_lo(v.z) * scale, bf16_hi(v.z) * scale);
      b[3] = e4m3x2(bf16_lo(v.w) * scale, bf16_hi(v.w) * scale);
      if (q) *reinterpret_cast<uint2*>(q + r * cols + c) = make_uint2(b[0] | (b[1] << 16), b[2] | (b[3] << 16));
    }
    if (q_t) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tile[cchunk * 8 + 2 * e][lr] = (uint8_t)(b[e] & 0xFF);
        tile[cchunk * 8 + 2 * e + 1][lr] = (uint8_t)(b[e] >> 8);
      }
    }
  }
  if (q_t) {
    __syncthreads();
    // thread -> one column, 32 consecutive positions (2 x 16 bytes) of the transposed copy
    const int lc = t >> 2, seg = (t & 3) * 32;
    const int64_t c = c0 + lc;
    if (c < cols) {
      const uint4 lo = *reinterpret_cast<const uint4*>(&tile[lc][seg]);
      const uint4 hi = *reinterpret_cast<const uint4*>(&tile[lc][seg + 16]);
      uint8_t* dst = q_t + c * ld_t + p0 + seg;
      *reinterpret_cast<uint4*>(dst) = lo;
      *reinterpret_cast<uint4*>(dst + 16) = hi;
    }
  }
}

hipError_t launch_quantize_fp8_grouped(const uint16_t* src, int64_t rows, int64_t cols, int G,
                                       const int64_t* layout, int64_t ld_t, float* amax_ws, const float* amax_in,
                                       uint8_t* q, uint8_t* q_t, float* amax, float* scale, float* scale_inv,
                                       hipStream_t s) {
  const int64_t npos = layout ? ld_t : rows;            // positions the tiles walk (a bound of the last group's end)
  hipError_t e = hipSuccess;
  const float* amax_g = amax_in;
  if (!amax_in) {                                       // the amax pass (skipped when the producer reduced it)
    if ((e = launch_fill_f32_zero(amax_ws, G, s)) != hipSuccess) return e;
    const int64_t ta = (npos / kQR) * ((cols + kGAC - 1) / kGAC);
    if (ta > 0) {
      hipLaunchKernelGGL(amax_grouped_kernel, dim3((unsigned)ta), dim3(256), 0, s, src, rows, cols, G, layout,
                         amax_ws);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    amax_g = amax_ws;
  }
  int64_t tq = (npos / kQR) * ((cols + kQC - 1) / kQC);
  if (tq < 1) tq = 1;                                   // block 0 still writes every group's scales
  hipLaunchKernelGGL(quantize_fp8_grouped_kernel, dim3((unsigned)tq), dim3(256), 0, s, src, rows, cols, G, layout,
                     ld_t, amax_g, q, q_t, amax, scale, scale_inv);
  return hipGetLastError();
}

}  // namespace sge
