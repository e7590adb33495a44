// Device-side helpers shared by the gfx950 kernels of libsge.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sge {

typedef __attribute__((__ext_vector_type__(8))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

constexpr int kWave = 64;

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past num_records: the load returns zeros

// Buffer resource over [base, base + bytes); loads beyond it read as zero, stores beyond it are
// dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFF00 ? 0x7FFFFF00 : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t two) { return __builtin_bit_cast(float, two << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t two) { return __builtin_bit_cast(float, two & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }

// fp32 -> bf16 with round-to-nearest-even (the compiler's __bf16 conversion; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// fp32 -> OCP E4M3 byte: saturate to +-448 first, then the hardware round-to-nearest-even
// conversion (which alone turns overflow into NaN). Returns two bytes in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// ------------------------------------------------------------------- MXFP8
// E8M0 exponent of a block from its amax bit pattern (bf16 magnitude bits).
__device__ __forceinline__ int mx_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  const uint32_t f = amax_bits << 16;                  // as fp32 bits
  const int be = (int)(f >> 23);                       // biased exponent (0 for subnormals)
  int e;
  if (be > 0) {
    e = be - 127;
  } else {
    // subnormal: value = mant * 2^-149, floor(log2) = msb(mant) - 149
    e = (31 - __builtin_clz(f & 0x7FFFFFu)) - 149;
  }
  int x = e - 8;
  return x < -127 ? -127 : (x > 127 ? 127 : x);
}

// 2^-X as fp32 for X in [-127, 119] (always a normal number).
__device__ __forceinline__ float pow2_neg(int x) {
  return __builtin_bit_cast(float, (uint32_t)(127 - x) << 23);
}

// XOR swizzle of 16-byte chunks inside 128-byte LDS rows: rows r..r+7 (any 8
// consecutive rows) and rows 8 apart both land on distinct chunks, so the MFMA
// fragment reads and both tile-fill patterns are free of bank conflicts.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    T w = __shfl_xor(v, o, kWave);
    v = v > w ? v : w;
  }
  return v;
}

typedef int v4i __attribute__((__vector_size__(4 * sizeof(int))));
typedef int v2i __attribute__((__vector_size__(2 * sizeof(int))));

// ---------------------------------------------- MXFP8 with gfx950's scaled conversion
// v_cvt_scalef32_pk_fp8_bf16 converts two packed bf16 values to E4M3 divided by 2^E, where E is
// taken from the exponent field of its fp32 scale operand alone (E8M0: field 0 is 2^-127), with
// round-to-nearest-even, and turns magnitudes past 448 (after rounding) into 448 or NaN. Measured
// on MI355X over every bf16 pattern at 14 block exponents from -127 to 120 (the extremes, -126,
// -100, -20, -8, -1, 0, 1, 7, 8, 20, 100, 119): in range it matches the fp32 route (scale by
// 2^-X, clamp to +-448, v_cvt_pk_fp8_f32) bit for bit, so clamping the bf16 magnitudes to
// 448 * 2^X first makes the two routes agree on finite inputs; the quantizer tests compare
// every finite bf16 value against the oracle.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// The packed magnitude maximum of two bf16 lanes: per-half max of (v & 0x7FFF).
__device__ __forceinline__ uint32_t pk_absmax_bits(uint32_t m, uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, m),
                                                                __builtin_bit_cast(u16x2, v & 0x7FFF7FFFu)));
}
// bf16 bits of 448 * 2^X, the largest magnitude a block with exponent X encodes (X <= 119 for
// a finite block; larger X come only from Inf / NaN maxima and are held at 119).
__device__ __forceinline__ uint32_t mx_bound_bits(int X) { return ((uint32_t)((X > 119 ? 119 : X) + 135) << 7) | 0x60u; }
// Two packed bf16 with each magnitude clamped to its half of bound2, signs kept.
__device__ __forceinline__ uint32_t clamp_pair(uint32_t v, uint32_t bound2) {
  const u16x2 m = __builtin_elementwise_min(__builtin_bit_cast(u16x2, v & 0x7FFF7FFFu), __builtin_bit_cast(u16x2, bound2));
  return __builtin_bit_cast(uint32_t, m) | (v & 0x80008000u);
}
// The scale operand for block exponent X: E8M0 byte X + 127 in the fp32 exponent field.
__device__ __forceinline__ float mx_scale_operand(int X) { return __builtin_bit_cast(float, (uint32_t)(X + 127) << 23); }
// E4M3 codes of four values, packed bf16 pairs p01 (values 0, 1) and p23 (2, 3), already
// clamped, at block exponent given by `scale`: bytes 0..3 of the result.
__device__ __forceinline__ uint32_t e4m3x4_scaled(uint32_t p01, uint32_t p23, float scale) {
  s16x2 q = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(s16x2{0, 0}, __builtin_bit_cast(bf16x2v, p01), scale, false);
  q = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(q, __builtin_bit_cast(bf16x2v, p23), scale, true);
  return __builtin_bit_cast(uint32_t, q);
}

// MXFP8 of 8 bf16 values (one lane's 16 bytes, packed pairs) inside a block of 32 that four
// adjacent lanes (lane ^ 1, lane ^ 2) hold together: the block amax of the bf16 magnitudes,
// the E8M0 exponent, and this lane's 8 E4M3 codes (by the scaled conversion; the codes of
// the fp32 route for finite values). Every lane of the wave must take part.
__device__ __forceinline__ v2i mx_quant_lane8(const v4i& v, int& e8m0) {
  uint32_t m2 = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) m2 = pk_absmax_bits(m2, (uint32_t)v[e]);
  uint32_t m = (m2 & 0xFFFFu) > (m2 >> 16) ? (m2 & 0xFFFFu) : (m2 >> 16);
  uint32_t o = __shfl_xor(m, 1, 64);
  m = o > m ? o : m;
  o = __shfl_xor(m, 2, 64);
  m = o > m ? o : m;
  const int X = mx_exponent(m);
  const uint32_t bound = mx_bound_bits(X) * 0x10001u;
  const float sc = mx_scale_operand(X);
  e8m0 = X + 127;
  return v2i{(int)e4m3x4_scaled(clamp_pair((uint32_t)v[0], bound), clamp_pair((uint32_t)v[1], bound), sc),
             (int)e4m3x4_scaled(clamp_pair((uint32_t)v[2], bound), clamp_pair((uint32_t)v[3], bound), sc)};
}

}  // namespace sge
