// MFMA GEMM with scale / residual / SwiGLU epilogues for gfx950.
//
//   C[m][n] = epilogue( sum_k A[m][k] * B[n][k] )
//
// One kernel template covers the dense fused scaled linear (forward with the
// in-place residual add, dgrad and wgrad with alpha folded in) and the grouped
// linear (rows or the contraction partitioned by device-side group offsets).
// The forward with the residual as output is the fusion of "NVIDIA
// TransformerEngine Ops Fused Forward Linear Scale Add" (Description); alpha
// inside the backward GEMMs is "NVIDIA TransformerEngine Ops Fused Backward
// Linear Scale" (Description); the grouped schedules and the SwiGLU epilogues
// follow "Activation + GroupedLinear Fusion for MOE and other MOE
// optimizations" (Description, Sequence Diagram).
//
// Design (CDNA4):
// * 256 threads = 4 waves in a 2x2 grid; each wave owns WMF x WNF fragments of
//   32x32 fp32 accumulators (v_mfma_f32_32x32x16_bf16, or the MX-scaled
//   v_mfma_scale_f32_32x32x64_f8f6f4 for E4M3 / MXFP8 with E8M0 scales).
// * Tiles of 128 contraction bytes per row (64 bf16 or 128 fp8) are staged in
//   LDS, double-buffered, rows 128 B with an XOR swizzle of the 16-B chunks.
//   Global loads of tile k+1 are in flight while tile k is multiplied.
// * Operands stored contraction-contiguous are copied 16 B at a time; bf16
//   operands stored the other way round are loaded as 8x8 blocks and
//   transposed in registers on the way into LDS, so dgrad and wgrad read the
//   untransposed tensors directly.
// * The MFMA is issued with B as its first operand, so each lane ends with 4
//   consecutive output columns per group and stores 8 bytes of bf16 at a time.
#include "common.h"
#include "launch.h"

namespace sge {

enum { F_BF16 = 0, F_E4M3 = 1, F_MX = 2 };
enum { E_STORE = 0, E_SWIGLU = 1, E_DSWIGLU = 2 };
enum { S_DENSE = 0, S_GROUP_M = 1, S_GROUP_K = 2 };

constexpr int kRowBytes = 128;   // contraction bytes per LDS row and per k-tile

__device__ __forceinline__ uint32_t perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Transpose an 8x8 block of 16-bit values: in[i] holds row i (8 values, two per
// dword); out[j] receives column j.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint4& lo = in[2 * e];
      const uint4& hi = in[2 * e + 1];
      const uint32_t l = (j >> 1) == 0 ? lo.x : (j >> 1) == 1 ? lo.y : (j >> 1) == 2 ? lo.z : lo.w;
      const uint32_t h = (j >> 1) == 0 ? hi.x : (j >> 1) == 1 ? hi.y : (j >> 1) == 2 ? hi.z : hi.w;
      d[e] = perm(h, l, sel);
    }
    out[j] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Per-operand tile loader: global -> registers -> LDS.
template <int ROWS, bool KMAJ, int ES>
struct Loader {
  static constexpr int kRegs = KMAJ ? ROWS / 32 : 8;
  uint4 r[kRegs];

  // base: element (row, k) of the operand is at base[row*ld + k] (KMAJ) or
  // base[k*ld + row] (!KMAJ); rows >= row_end and k >= k_end read as zero.
  // rowmap: logical tile row -> operand row (identity except for SwiGLU).
  template <class RowMap>
  __device__ __forceinline__ void load(const uint8_t* __restrict__ base, int64_t ld, int64_t row0,
                                       int64_t row_end, int64_t k0, int64_t k_end,
                                       const RowMap& rowmap) {
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
      constexpr int kElemsPerChunk = 16 / ES;
      const int c = t & 7;
      const int64_t k = k0 + c * kElemsPerChunk;
#pragma unroll
      for (int i = 0; i < kRegs; ++i) {
        const int rr = (t >> 3) + 32 * i;
        const int64_t row = rowmap(row0, rr);
        if (row < row_end && k < k_end) {
          r[i] = *reinterpret_cast<const uint4*>(base + (row * ld + k) * ES);
        } else {
          r[i] = make_uint4(0, 0, 0, 0);
        }
      }
    } else {
      static_assert(ES == 2, "transposed tile loads exist for bf16 only");
      constexpr int kOuterChunks = ROWS / 8;
      if (t < ROWS) {
        const int oc = t % kOuterChunks;
        const int kc = t / kOuterChunks;
        const int64_t outer = row0 + oc * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int64_t k = k0 + kc * 8 + i;
          if (outer < row_end && k < k_end) {
            r[i] = *reinterpret_cast<const uint4*>(base + (k * ld + outer) * 2);
          } else {
            r[i] = make_uint4(0, 0, 0, 0);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t* lds) const {
    const int t = threadIdx.x;
    if constexpr (KMAJ) {
      const int c = t & 7;
#pragma unroll
      for (int i = 0; i < kRegs; ++i) {
        const int rr = (t >> 3) + 32 * i;
        *reinterpret_cast<uint4*>(lds + rr * kRowBytes + ((c ^ swz(rr)) << 4)) = r[i];
      }
    } else {
      constexpr int kOuterChunks = ROWS / 8;
      if (t < ROWS) {
        const int oc = t % kOuterChunks;
        const int kc = t / kOuterChunks;
        uint4 tr[8];
        transpose8x8(r, tr);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int rr = oc * 8 + j;
          *reinterpret_cast<uint4*>(lds + rr * kRowBytes + ((kc ^ swz(rr)) << 4)) = tr[j];
        }
      }
    }
  }
};

struct IdentityRows {
  __device__ __forceinline__ int64_t operator()(int64_t row0, int rr) const { return row0 + rr; }
};

// SwiGLU pairing: the B tile's rows are, per wave column, `half` gate rows of
// W followed by the matching `half` rows of the up projection (offset F), so
// fragment j and j + WNF/2 of a wave hold a and b of the same output column.
template <int WN>
struct SwigluRows {
  int64_t F;
  __device__ __forceinline__ int64_t operator()(int64_t col0, int rr) const {
    constexpr int half = WN / 2;
    const int wn = rr / WN;
    const int r = rr % WN;
    const int64_t base = col0 + wn * half;
    return r < half ? base + r : F + base + (r - half);
  }
};

template <int FMT, bool AK, bool BK, int EPI, int SCHED, int WMF, int WNF>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void gemm_kernel(const GemmParams p) {
  constexpr int ES = FMT == F_BF16 ? 2 : 1;
  constexpr int WM = 32 * WMF, WN = 32 * WNF;
  constexpr int BM = 2 * WM, BN = 2 * WN;
  constexpr int KT_ELEMS = kRowBytes / ES;               // contraction elements per k-tile
  constexpr int A_BYTES = BM * kRowBytes, B_BYTES = BN * kRowBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_BYTES + B_BYTES)];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---------------------------------------------------------------- schedule
  int64_t m0, n0, row_end, k_begin = 0, k_end = p.K;
  const uint8_t* bptr = p.b;
  uint16_t* cptr = p.c;
  int nt;
  if constexpr (SCHED == S_DENSE) {
    int bid = blockIdx.x;
    const int nblk = gridDim.x;
    if ((nblk & 7) == 0) bid = (bid & 7) * (nblk >> 3) + (bid >> 3);   // tiles of one XCD adjacent
    const int MT = p.mt_count, NT = p.nt_count;
    const int GM = 8;
    const int group = bid / (GM * NT);
    const int first_m = group * GM;
    const int gsz = min(MT - first_m, GM);
    const int in_group = bid % (GM * NT);
    const int mt = first_m + in_group % gsz;
    nt = in_group / gsz;
    m0 = (int64_t)mt * BM;
    n0 = (int64_t)nt * BN;
    row_end = p.M;
  } else if constexpr (SCHED == S_GROUP_M) {
    nt = blockIdx.x % p.nt_count;
    int lin = blockIdx.x / p.nt_count;
    int g = -1;
    int64_t lo = 0, hi = 0, prev = 0;
    for (int gg = 0; gg < p.G; ++gg) {
      int64_t a = p.offsets[gg], b = p.offsets[gg + 1];
      a = a < prev ? prev : (a > p.T ? p.T : a);
      b = b < a ? a : (b > p.T ? p.T : b);
      prev = b;
      const int tiles = (int)((b - a + BM - 1) / BM);
      if (lin < tiles) { g = gg; lo = a; hi = b; break; }
      lin -= tiles;
    }
    if (g < 0) return;                                   // beyond the last real tile
    m0 = lo + (int64_t)lin * BM;
    row_end = hi;
    n0 = (int64_t)nt * (EPI == E_SWIGLU ? BN / 2 : BN);
    bptr += (int64_t)g * p.b_group_stride * ES;
  } else {
    const int per = p.mt_count * p.nt_count;
    const int g = blockIdx.x / per;
    const int rem = blockIdx.x % per;
    const int mt = rem / p.nt_count;
    nt = rem % p.nt_count;
    int64_t prev = 0, a = 0, b = 0;
    for (int gg = 0; gg <= g; ++gg) {
      a = p.offsets[gg];
      b = p.offsets[gg + 1];
      a = a < prev ? prev : (a > p.T ? p.T : a);
      b = b < a ? a : (b > p.T ? p.T : b);
      prev = b;
    }
    k_begin = a;
    k_end = b;
    m0 = (int64_t)mt * BM;
    n0 = (int64_t)nt * BN;
    row_end = p.M;
    cptr += (int64_t)g * p.c_group_stride;
  }
  const int64_t n_end = EPI == E_SWIGLU ? p.F : p.N;

  // ---------------------------------------------------------------- main loop
  f32x16 acc[WMF][WNF];
#pragma unroll
  for (int i = 0; i < WMF; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  Loader<BM, AK, ES> la;
  Loader<BN, BK, ES> lb;
  IdentityRows idrows;
  SwigluRows<WN> swrows{p.F};
  // Rows of B beyond the operand: N (dense / group M), or N_out rows for group K.
  const int64_t b_rows = EPI == E_SWIGLU ? 2 * p.F : p.N;

  auto load_tiles = [&](int64_t k0) {
    la.load(p.a, p.lda, m0, row_end, k0, k_end, idrows);
    if constexpr (EPI == E_SWIGLU) lb.load(bptr, p.ldb, n0, b_rows, k0, k_end, swrows);
    else lb.load(bptr, p.ldb, n0, b_rows, k0, k_end, idrows);
  };

  // MX scales: one dword per fragment row holds the 4 E8M0 bytes of a k-tile,
  // pre-shifted so byte 2*ks of the register is this lane's 32-block.
  uint32_t sa[WMF], sb[WNF];
  auto load_scales = [&](int64_t k0) {
    if constexpr (FMT == F_MX) {
      const int64_t blk0 = k0 >> 5;
      const int64_t nblk = (k_end + 31) >> 5;
      const int sh = 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < WMF; ++i) {
        const int64_t row = m0 + wm * WM + i * 32 + (lane & 31);
        uint32_t v = 0x7F7F7F7Fu;
        if (row < row_end) {
          const uint8_t* s = p.a_mx + row * p.a_mx_ld + blk0;
          if (p.mx_aligned) {
            v = *reinterpret_cast<const uint32_t*>(s);
          } else {
            v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) v |= (blk0 + e < nblk ? (uint32_t)s[e] : 127u) << (8 * e);
          }
        }
        sa[i] = v >> sh;
      }
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        const int64_t row = n0 + wn * WN + j * 32 + (lane & 31);
        uint32_t v = 0x7F7F7F7Fu;
        if (row < b_rows) {
          const uint8_t* s = p.b_mx + row * p.b_mx_ld + blk0;
          if (p.mx_aligned) {
            v = *reinterpret_cast<const uint32_t*>(s);
          } else {
            v = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) v |= (blk0 + e < nblk ? (uint32_t)s[e] : 127u) << (8 * e);
          }
        }
        sb[j] = v >> sh;
      }
    }
  };

  const int64_t klen = k_end - k_begin;
  const int KT = klen > 0 ? (int)((klen + KT_ELEMS - 1) / KT_ELEMS) : 0;

  if (KT > 0) {
    load_tiles(k_begin);
    la.store(smem);
    lb.store(smem + A_BYTES);
    __syncthreads();
  }

  const int lrow = lane & 31;
  const int lhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    uint8_t* a_lds = smem + (kt & 1) * (A_BYTES + B_BYTES);
    uint8_t* b_lds = a_lds + A_BYTES;
    const bool more = kt + 1 < KT;
    const int64_t k0 = k_begin + (int64_t)kt * KT_ELEMS;
    load_scales(k0);
    if (more) load_tiles(k0 + KT_ELEMS);

    if constexpr (FMT == F_BF16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = ks * 2 + lhalf;
        bf16x8 af[WMF], bfr[WNF];
#pragma unroll
        for (int i = 0; i < WMF; ++i) {
          const int r = wm * WM + i * 32 + lrow;
          af[i] = *reinterpret_cast<const bf16x8*>(a_lds + r * kRowBytes + ((ch ^ swz(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
          const int r = wn * WN + j * 32 + lrow;
          bfr[j] = *reinterpret_cast<const bf16x8*>(b_lds + r * kRowBytes + ((ch ^ swz(r)) << 4));
        }
#pragma unroll
        for (int i = 0; i < WMF; ++i)
#pragma unroll
          for (int j = 0; j < WNF; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // f8f6f4 32x32x64 lane layout: bytes 0-15 hold k = 16*half .. +15 and
        // bytes 16-31 hold k = 32 + 16*half .. +15 of the 64-wide step.
        const int c0 = ks * 4 + lhalf, c1 = c0 + 2;
        i32x8 af[WMF], bfr[WNF];
#pragma unroll
        for (int i = 0; i < WMF; ++i) {
          const int r = wm * WM + i * 32 + lrow;
          const uint8_t* row = a_lds + r * kRowBytes;
          const int4 lo = *reinterpret_cast<const int4*>(row + ((c0 ^ swz(r)) << 4));
          const int4 hi = *reinterpret_cast<const int4*>(row + ((c1 ^ swz(r)) << 4));
          af[i] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
#pragma unroll
        for (int j = 0; j < WNF; ++j) {
          const int r = wn * WN + j * 32 + lrow;
          const uint8_t* row = b_lds + r * kRowBytes;
          const int4 lo = *reinterpret_cast<const int4*>(row + ((c0 ^ swz(r)) << 4));
          const int4 hi = *reinterpret_cast<const int4*>(row + ((c1 ^ swz(r)) << 4));
          bfr[j] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        }
#pragma unroll
        for (int i = 0; i < WMF; ++i)
#pragma unroll
          for (int j = 0; j < WNF; ++j) {
            if constexpr (FMT == F_MX) {
              if (ks == 0)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bfr[j], af[i], acc[i][j], 0, 0, 0, (int)sb[j], 0, (int)sa[i]);
              else
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    bfr[j], af[i], acc[i][j], 0, 0, 2, (int)sb[j], 2, (int)sa[i]);
            } else {
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bfr[j], af[i], acc[i][j], 0, 0, 0, 0x7F7F7F7F, 0, 0x7F7F7F7F);
            }
          }
      }
    }

    if (more) {
      uint8_t* na = smem + ((kt + 1) & 1) * (A_BYTES + B_BYTES);
      la.store(na);
      lb.store(na + A_BYTES);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  float alpha = p.alpha;
  if constexpr (FMT == F_E4M3) alpha = (p.a_sinv[0] * p.b_sinv[0]) * p.alpha;

  if constexpr (EPI == E_STORE) {
#pragma unroll
    for (int i = 0; i < WMF; ++i) {
      const int64_t m = m0 + wm * WM + i * 32 + lrow;
      if (m >= row_end) continue;
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = n0 + wn * WN + j * 32 + 8 * q + 4 * lhalf;
          if (n >= n_end) continue;
          float v0 = alpha * acc[i][j][4 * q + 0], v1 = alpha * acc[i][j][4 * q + 1];
          float v2 = alpha * acc[i][j][4 * q + 2], v3 = alpha * acc[i][j][4 * q + 3];
          uint16_t* cp = cptr + m * p.ldc + n;
          if (p.accumulate) {
            const uint2 r = *reinterpret_cast<const uint2*>(cp);
            v0 = bf16_lo(r.x) + v0;
            v1 = bf16_hi(r.x) + v1;
            v2 = bf16_lo(r.y) + v2;
            v3 = bf16_hi(r.y) + v3;
          }
          *reinterpret_cast<uint2*>(cp) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
        }
      }
    }
  } else if constexpr (EPI == E_SWIGLU) {
    constexpr int HJ = WNF / 2;
#pragma unroll
    for (int i = 0; i < WMF; ++i) {
      const int64_t m = m0 + wm * WM + i * 32 + lrow;
      if (m >= row_end) continue;
      const float pm = p.probs[m];
#pragma unroll
      for (int j = 0; j < HJ; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = n0 + wn * (WN / 2) + j * 32 + 8 * q + 4 * lhalf;
          if (col >= n_end) continue;
          float a[4], b[4], y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = alpha * acc[i][j][4 * q + e];
            b[e] = alpha * acc[i][j + HJ][4 * q + e];
            y[e] = pm * (a[e] * fast_sigmoid(a[e])) * b[e];
          }
          if (p.aux) {
            uint16_t* hp = p.aux + m * p.ld_aux + col;
            *reinterpret_cast<uint2*>(hp) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
            *reinterpret_cast<uint2*>(hp + p.F) =
                make_uint2(pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]));
          }
          *reinterpret_cast<uint2*>(cptr + m * p.ldc + col) =
              make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        }
      }
    }
  } else {  // E_DSWIGLU
#pragma unroll
    for (int i = 0; i < WMF; ++i) {
      const int64_t m = m0 + wm * WM + i * 32 + lrow;
      const bool mok = m < row_end;
      const float pm = mok ? p.probs[m] : 0.0f;
      float part = 0.0f;
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = n0 + wn * WN + j * 32 + 8 * q + 4 * lhalf;
          if (!mok || n >= n_end) continue;
          const uint16_t* hp = p.aux + m * p.ld_aux + n;
          const uint2 ha = *reinterpret_cast<const uint2*>(hp);
          const uint2 hb = *reinterpret_cast<const uint2*>(hp + p.F);
          const float a[4] = {bf16_lo(ha.x), bf16_hi(ha.x), bf16_lo(ha.y), bf16_hi(ha.y)};
          const float b[4] = {bf16_lo(hb.x), bf16_hi(hb.x), bf16_lo(hb.y), bf16_hi(hb.y)};
          float da[4], db[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = alpha * acc[i][j][4 * q + e];
            const float s = fast_sigmoid(a[e]);
            const float silu = a[e] * s;
            const float dsilu = s * (1.0f + a[e] * (1.0f - s));
            da[e] = g * pm * b[e] * dsilu;
            db[e] = g * pm * silu;
            part += g * silu * b[e];
          }
          uint16_t* dp = p.aux_out + m * p.ld_aux_out + n;
          *reinterpret_cast<uint2*>(dp) = make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
          *reinterpret_cast<uint2*>(dp + p.F) =
              make_uint2(pack_bf16x2(db[0], db[1]), pack_bf16x2(db[2], db[3]));
        }
      }
      part += __shfl_xor(part, 32, 64);
      if (mok && lhalf == 0) p.dp_part[(int64_t)(nt * 2 + wn) * p.T + m] = part;
    }
  }
}

// ------------------------------------------------------------------ launchers
template <int FMT, bool AK, bool BK, int EPI, int SCHED, int WMF, int WNF>
static hipError_t launch_cfg(GemmParams p, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<FMT, AK, BK, EPI, SCHED, WMF, WNF>), dim3(grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int FMT, bool AK, bool BK, int EPI, int SCHED>
static hipError_t launch_tile(GemmParams p, hipStream_t s) {
  constexpr int WMF = 4, WNF = 4;
  constexpr int BM = 64 * WMF, BN = 64 * WNF;
  int grid = 0;
  if constexpr (SCHED == S_DENSE) {
    p.mt_count = (int)((p.M + BM - 1) / BM);
    p.nt_count = (int)((p.N + BN - 1) / BN);
    grid = p.mt_count * p.nt_count;
  } else if constexpr (SCHED == S_GROUP_M) {
    const int64_t ncols = EPI == E_SWIGLU ? p.F : p.N;
    const int64_t ntile = EPI == E_SWIGLU ? BN / 2 : BN;
    p.nt_count = (int)((ncols + ntile - 1) / ntile);
    const int64_t mtiles = (p.T + BM - 1) / BM + p.G;     // upper bound over any split
    grid = (int)(mtiles * p.nt_count);
  } else {
    p.mt_count = (int)((p.M + BM - 1) / BM);
    p.nt_count = (int)((p.N + BN - 1) / BN);
    grid = p.mt_count * p.nt_count * p.G;
  }
  return launch_cfg<FMT, AK, BK, EPI, SCHED, WMF, WNF>(p, grid, s);
}

hipError_t launch_gemm(const GemmParams& p, int fmt, bool a_kmaj, bool b_kmaj, hipStream_t s) {
  if (fmt == F_BF16) {
    if (a_kmaj && b_kmaj) return launch_tile<F_BF16, true, true, E_STORE, S_DENSE>(p, s);
    if (a_kmaj && !b_kmaj) return launch_tile<F_BF16, true, false, E_STORE, S_DENSE>(p, s);
    if (!a_kmaj && !b_kmaj) return launch_tile<F_BF16, false, false, E_STORE, S_DENSE>(p, s);
    return launch_tile<F_BF16, false, true, E_STORE, S_DENSE>(p, s);
  }
  if (fmt == F_E4M3) return launch_tile<F_E4M3, true, true, E_STORE, S_DENSE>(p, s);
  return launch_tile<F_MX, true, true, E_STORE, S_DENSE>(p, s);
}

hipError_t launch_grouped_fwd(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_SWIGLU) return launch_tile<F_BF16, true, true, E_SWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_BF16, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_dgrad(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_DSWIGLU) return launch_tile<F_BF16, true, false, E_DSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_BF16, true, false, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_wgrad(const GemmParams& p, hipStream_t s) {
  return launch_tile<F_BF16, false, false, E_STORE, S_GROUP_K>(p, s);
}

int gemm_tile_n() { return 256; }

}  // namespace sge
