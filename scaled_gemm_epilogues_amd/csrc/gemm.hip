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
// * 256x256 macro tiles: 8 waves in a 2x4 grid (bf16, E4M3) or 4 waves in a 2x2 grid
//   (MXFP8); each wave owns WMF x WNF blocks of 32x32 fp32 accumulators, multiplied with
//   v_mfma_f32_16x16x32_bf16 (four per block and k-step) for bf16, or with the MX-scaled
//   v_mfma_scale_f32_32x32x64_f8f6f4 for E4M3 / MXFP8 with E8M0 scales.
// * Tiles are renumbered so each XCD runs a contiguous block of them (its own L2).
// * Tiles of 128 contraction bytes per operand row (64 bf16 or 128 fp8) move
//   from HBM straight into LDS with buffer_load ... lds (no staging registers;
//   out-of-range lanes read zeros), in two LDS stages (8-bit dense and weight-gradient
//   GEMMs: four stages of 64 bytes): the copy of a later tile is in flight while a
//   tile is multiplied. LDS images are laid out (XOR-swizzled 16-B chunks, 16-row
//   blocks for bf16) so fragment reads are free of bank conflicts.
// * bf16 operands stored with the contraction dimension outermost (dgrad's W,
//   wgrad's dy and x) are copied as they are and read with the transposing
//   ds_read_b64_tr_b16, so dgrad and wgrad read the untransposed tensors.
// * Fragments of the next k-step are read from LDS while the MFMAs of the current one run.
// * The MFMA is issued with B as its first operand, so each lane ends with 4
//   consecutive output columns per group and stores 8 bytes of bf16 at a time.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace sge {

enum { F_BF16 = 0, F_E4M3 = 1, F_MX = 2, F_MXU = 3 };   // F_MXU: MXFP8 with unaligned scale rows
enum { E_STORE = 0, E_SWIGLU = 1, E_DSWIGLU = 2, E_SRELU = 3, E_DSRELU = 4, E_CSWIGLU = 5, E_DCSWIGLU = 6 };
// Gated forward epilogues: B's rows are the gate / up halves interleaved per tile, output F wide.
constexpr bool glu_fwd(int e) { return e == E_SWIGLU || e == E_CSWIGLU; }
enum { S_DENSE = 0, S_GROUP_M = 1, S_GROUP_K = 2 };

constexpr int kRowBytes = 128;   // contraction bytes per LDS row and per k-tile

// Macro tile 256x256. bf16 and E4M3: 2x4 waves (two per SIMD), each owning 4x2 32x32
// accumulator blocks, so one wave's LDS and barrier waits are covered by the other's MFMAs.
// MXFP8 (more live registers for the E8M0 scales): 2x2 waves, each 4x4 accumulators.
#ifndef SGE_WAVES_M
#define SGE_WAVES_M 2
#define SGE_WAVES_N 4
#define SGE_FRAGS_M 4
#define SGE_FRAGS_N 2
#endif
constexpr int kWavesM = SGE_WAVES_M, kWavesN = SGE_WAVES_N, kFragsM = SGE_FRAGS_M, kFragsN = SGE_FRAGS_N;
#ifndef SGE_XCD_GROUP_M
#define SGE_XCD_GROUP_M 4
#endif
#ifndef SGE_GROUPED_GM
#define SGE_GROUPED_GM 4         // row tiles per band in a group's tile order (grouped rows)
#endif
#ifndef SGE_GROUPED_GM_STORE
#define SGE_GROUPED_GM_STORE 8   // the same for plain-store launches with a K-major weight
#endif
#ifndef SGE_RD_PER_MFMA
#define SGE_RD_PER_MFMA 2        // fragment reads issued after each MFMA (bf16, E4M3)
#endif
#ifndef SGE_RD_PER_MFMA_MX
#define SGE_RD_PER_MFMA_MX 1     // the same for MXFP8 (one read per MFMA: 7% faster step than two)
#endif
#ifndef SGE_RD_PER_MFMA_GROUPED
#define SGE_RD_PER_MFMA_GROUPED 1  // bf16 / E4M3 grouped schedules (1% faster bf16 grouped MLP)
#endif
#ifndef SGE_DSWIGLU_BATCH
#define SGE_DSWIGLU_BATCH 4      // dSwiGLU epilogue chunks whose loads are in flight together
#endif

#ifndef SGE_BF16_M16
#define SGE_BF16_M16 1           // bf16 tiles multiply with 16x16x32 MFMAs (else 32x32x16)
#endif

#ifndef SGE_M16_CPG
#define SGE_M16_CPG 2            // bf16 16x16x32 loop: tile copies issued after each MFMA group (1, 4 and 8 measured slower)
#endif

#ifndef SGE_DEEP_8BIT
#define SGE_DEEP_8BIT 1          // 8-bit dense / weight-gradient GEMMs: 64-byte k-tiles, four LDS stages
#endif

// Deep pipeline: with one wave per SIMD nothing covers a wave's wait for its tile copies, so the
// 8-bit dense GEMMs keep four k-tiles of copies in flight (four LDS stages of 64 contraction
// bytes, one MFMA k-step each, 128 KB in all) instead of one (two stages of 128 bytes). The bf16
// tiles keep two stages and two waves per SIMD: four 32- or 64-byte stages (a barrier every k-step)
// and 2x2-wave tiles measured 4-30% slower on 32x32x16 MFMAs and 12-15% slower on 16x16x32 ones.
// Among the grouped GEMMs only the weight gradients (contraction over a group's tokens: few,
// long tiles) take it: measured on the FP8 / MXFP8 grouped MLP they ran 2.5-4.6% faster, while
// the row-partitioned ones ran from 2% faster to 29% slower (the FP8 activation-backward
// epilogue on four waves instead of eight).
constexpr bool deep_pipe(int fmt, int sched, int epi) {
  return SGE_DEEP_8BIT && (fmt == F_MX || fmt == F_E4M3) && (sched == S_DENSE || sched == S_GROUP_K) &&
         epi == E_STORE;
}

// Waves and fragments of a tile: MXFP8 (more live registers for the E8M0 scales) and the
// deep-pipelined 8-bit tiles take 2x2 waves of 4x4 accumulators (one wave per SIMD; a third
// fewer LDS fragment bytes per MFMA); the rest 2x4 waves of 4x2.
template <int FMT, int SCHED, int EPI>
struct TileShape {
  static constexpr bool k4 = FMT == F_MX || FMT == F_MXU || deep_pipe(FMT, SCHED, EPI);
  static constexpr int WGM = k4 ? 2 : kWavesM, WGN = k4 ? 2 : kWavesN;
  static constexpr int WMF = k4 ? 4 : kFragsM, WNF = k4 ? 4 : kFragsN;
};

// The dispatcher hands workgroups to the 8 XCDs round-robin (workgroup b runs on XCD b % 8),
// and each XCD has its own L2. Renumbering so that XCD x receives one contiguous range of
// tile indices makes the tiles an XCD runs at the same time neighbours, sharing operand
// panels in its L2. Bijective on [0, total) for any total.
__device__ __forceinline__ int xcd_tile(int bid, int total) {
  const int x = bid & 7, i = bid >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + i;
}

__device__ __forceinline__ float fast_sigmoid(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Per-group amax of an epilogue's bf16 output: each wave folds the max of its fp32 values
// (before their bf16 rounding: rounding is monotone, so the rounded max is the max of the
// stored values) into a workgroup LDS slot, as bf16 bits << 16, i.e. the value as fp32;
// non-negative floats order like their bit patterns. One global atomic per workgroup.
__device__ __forceinline__ void amax_to_slot(uint32_t* slot, float m) {
  uint32_t b = (uint32_t)f32_to_bf16(m) << 16;
  b = wave_max(b);
  if ((threadIdx.x & 63) == 0 && b) atomicMax(slot, b);
}
__device__ __forceinline__ void slot_to_group(uint32_t* slot, float* amax, int g) {
  __syncthreads();
  if (threadIdx.x == 0 && *slot) atomicMax(reinterpret_cast<uint32_t*>(amax) + g, *slot);
}


typedef short i16x4 __attribute__((__vector_size__(4 * sizeof(short))));


// The same resource as four dwords, for the direct-to-LDS copies issued from inline asm.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc4(const void* base, int64_t bytes) {
  const int n = bytes > 0x7FFFFF00 ? 0x7FFFFF00 : (bytes < 0 ? 0 : (int)bytes);
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), n, 0x00020000};
}

// buffer_load_dwordx4 ... lds: lane i's 16 bytes at voff land at LDS byte lds_addr + 16*i
// (lds_addr wave-uniform). Issued from asm so that the compiler tracks no LDS writes in
// flight: it would otherwise make reads of the stage being multiplied wait for the copy
// into the other stage (it cannot always tell the two apart). Completion is the caller's
// explicit s_waitcnt vmcnt plus the workgroup barrier before a stage is read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(const i32x4& rsrc, const void* lds, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
  // wave-uniform by construction; readfirstlane states it so the descriptor sits in SGPRs
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rsrc.x), __builtin_amdgcn_readfirstlane(rsrc.y),
                   __builtin_amdgcn_readfirstlane(rsrc.z), __builtin_amdgcn_readfirstlane(rsrc.w)};
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(voff), "s"(r)
               : "memory", "m0");
}
// The same with the LDS byte address given as a wave-uniform 32-bit value (kept in SGPRs).
__device__ __forceinline__ void lds_copy16_at(const i32x4& rsrc, uint32_t lds_addr, uint32_t voff) {
  const i32x4 r = {__builtin_amdgcn_readfirstlane(rsrc.x), __builtin_amdgcn_readfirstlane(rsrc.y),
                   __builtin_amdgcn_readfirstlane(rsrc.z), __builtin_amdgcn_readfirstlane(rsrc.w)};
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(lds_addr)),
               "v"(voff), "s"(r)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// XOR swizzle of the 16-byte chunks of an LDS row: 128-byte rows use swz(); 64-byte rows (four
// chunks) flip by (row / 4) % 4, so 16 consecutive rows reading one logical chunk (a phase of a
// ds_read_b128) cover all 64 banks.
template <int RB>
__device__ __forceinline__ int swz_rows(int row) {
  if constexpr (RB == 128) return swz(row);
  else return (row >> 2) & 3;
}

// 16-byte chunk swizzle of contraction row k of an outer-contiguous bf16 tile (512-byte rows): bits
// 2-3 from k % 4 spread the four rows one transposing read covers; with 16x16x32 MFMAs the four
// 16-lane groups read rows k, k + 8, k + 16 and k + 24 (32 bytes each), which bits 1 and 4 (from
// k / 8 and k / 16) also spread. The weight-gradient GEMM, whose fragments all come from such
// reads, shows no LDS bank conflicts on MI355X (SQ_LDS_BANK_CONFLICT) beyond its epilogue's.
__device__ __forceinline__ int tr_swz(int k) {
  return 4 * (k & 3) ^ (SGE_BF16_M16 ? 2 * ((k >> 3) & 1) ^ 16 * ((k >> 4) & 1) : 0);
}
// Inner-contiguous bf16 tiles under 16x16x32 MFMAs are stored in 1-KB blocks: block b holds rows
// 16 (b / 2) .. + 15 at contraction bytes 64 (b % 2) .. + 63 (one k-step), row i of the block at
// byte 64 i, its 16-byte chunk c at slot c ^ ((i / 2) % 4). A fragment read (lane l: row l % 16,
// chunk l / 16) then takes one block; measured on MI355X (LDS timing and SQ_LDS_BANK_CONFLICT) it
// runs conflict-free, as fast as the 32x32x16 reads of 128-byte rows, while reading 128-byte rows
// at chunks l / 16 costs 4 extra cycles per read under every XOR swizzle of the chunks tried. The
// copy of a block stays coalesced: lanes 4i .. 4i + 3 fetch the 64 contiguous bytes of row i.
__device__ __forceinline__ int blk16_slot(int i, int c) { return c ^ ((i >> 1) & 3); }

// Global -> LDS copy of one operand tile with buffer_load ... lds (16 B per lane, the wave's
// 64 lanes filling 1 KB of LDS contiguously); no staging registers. Lanes fetch permuted
// sources so that the LDS image is swizzled:
// * inner-contiguous tile: ROWS rows of 128 contraction bytes; chunk c of row r sits at
//   chunk c ^ swz(r) (8-bit), or in the 16-row blocks of blk16_slot (bf16);
// * outer-contiguous tile (bf16): 64 contraction rows of ROWS*2 bytes; chunk c of row k sits
//   at chunk c ^ tr_swz(k), so the 32 lanes the LDS serves per cycle for a transposing
//   ds_read_b64_tr_b16 hit distinct banks.
// Chunks outside the operand (rows >= row_end, contraction >= k_end) are fetched from an
// out-of-range offset and land as zeros.
template <int ROWS, bool KMAJ, int ES, int NWAVES, int RB = kRowBytes>
struct TileCopy {
  static constexpr int kInstr = ROWS * RB / 1024 / NWAVES;          // 1-KB pieces per wave
  static constexpr int kRowsPerInstr = KMAJ ? 1024 / RB : 1024 / (ROWS * 2);
  static constexpr int kChunksPerRow = KMAJ ? RB / 16 : ROWS / 8;
  uint32_t off[kInstr];      // byte offset of the lane's source at contraction 0 (or kOOB)
  int32_t kk[kInstr];        // contraction index of the lane's source relative to the tile start

  template <class RowMap>
  __device__ __forceinline__ void init(int64_t ld, int64_t row0, int64_t row_end, const RowMap& rowmap) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int piece = NWAVES * i + wave;
      const int r = piece * kRowsPerInstr + lane / kChunksPerRow;   // LDS row
      const int p = lane % kChunksPerRow;                           // physical chunk
      if constexpr (KMAJ) {
        if constexpr (ES == 2 && SGE_BF16_M16) {
          static_assert(RB == 128 && ROWS % 16 == 0, "16-row blocks of two 64-byte halves");
          const int rb = (piece >> 1) * 16 + (lane >> 2);                 // row of this lane's chunk
          const int cb = 4 * (piece & 1) + blk16_slot(lane >> 2, lane & 3);
          const int64_t row = rowmap(row0, rb);
          kk[i] = cb * 8;
          off[i] = row < row_end ? (uint32_t)((row - row0) * ld * 2 + cb * 16) : kOOB;
        } else {
        const int c = p ^ swz_rows<RB>(r);
        const int64_t row = rowmap(row0, r);
        kk[i] = c * (16 / ES);
        off[i] = row < row_end ? (uint32_t)((row - row0) * ld * ES + c * 16) : kOOB;
        }
      } else {
        const int c = p ^ tr_swz(r);
        const int64_t outer = row0 + c * 8;
        kk[i] = r;
        off[i] = outer < row_end ? (uint32_t)(r * ld * 2 + c * 16) : kOOB;
      }
    }
  }

  // Issue the copy of contraction range [k0, k0 + tile) into lds (base of this operand's tile).
  // base_row0: address of operand row row0 (inner-contiguous) or of contraction row 0 (outer).
  __device__ __forceinline__ void issue(uint8_t* lds, const uint8_t* base, int64_t ld, int64_t bytes_from_base,
                                        int64_t k0, int64_t k_end) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Resource based at the tile's first contraction element keeps offsets 32-bit.
    const int64_t shift = KMAJ ? k0 * ES : k0 * ld * 2;
    const i32x4 rsrc = make_rsrc4(base + shift, bytes_from_base - shift);
    const int64_t kl = k_end - k0;                       // chunks at or past it read zeros
    const int klim = kl < (1 << 30) ? (int)kl : (1 << 30);
    const uint32_t dst = lds_addr_of(lds);
#pragma unroll
    for (int i = 0; i < kInstr; ++i) lds_copy16_at(rsrc, dst + (uint32_t)((NWAVES * i + wave) * 1024), kk[i] < klim ? off[i] : kOOB);
  }
};

// bf16 MFMA fragment (8 contraction values of one row) from an inner-contiguous tile.
__device__ __forceinline__ bf16x8 frag_k_bf16(const uint8_t* lds, int r, int ch) {
  return *reinterpret_cast<const bf16x8*>(lds + r * kRowBytes + ((ch ^ swz(r)) << 4));
}
// The 16x16x32 fragment (lane l: row rbase + l % 16, contraction 32 ks + 8 (l / 16) .. + 7) from
// an inner-contiguous tile in 16-row blocks (rbase % 16 == 0).
__device__ __forceinline__ bf16x8 frag_k16_bf16(const uint8_t* lds, int rbase, int ks, int lane) {
  const int i = lane & 15;
  return *reinterpret_cast<const bf16x8*>(lds + (rbase >> 4) * 2048 + ks * 1024 + i * 64 +
                                          (blk16_slot(i, lane >> 4) << 4));
}

// The same fragment from an outer-contiguous tile with two transposing reads. Within each
// 16-lane group, ds_read_b64_tr_b16 hands output lane 4g+c element c of the 8-byte rows
// addressed by lanes g, 4+g, 8+g, 12+g; lane s therefore addresses contraction row
// kb + s/4 at outer offset 4*(s%4), and output lane i receives rows kb..kb+3 of outer i.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_t_bf16(const uint8_t* lds, int mbase, int ks, int lane) {
  const int q = lane >> 4, s = lane & 15;
  const int m = mbase + 16 * (q & 1) + 4 * (s & 3);
  const int k = ks * 16 + 8 * (q >> 1) + (s >> 2);
  const int k2 = k + 4;
  const uint8_t* p0 = lds + k * (ROWS * 2) + (((m >> 3) ^ tr_swz(k)) << 4) + (m & 7) * 2;
  const uint8_t* p1 = lds + k2 * (ROWS * 2) + (((m >> 3) ^ tr_swz(k2)) << 4) + (m & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
  typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// The 16x16x32 operand fragment (lane l: outer mbase + l % 16, contraction 32 ks + 8 (l / 16) ..
// + 7) from an outer-contiguous tile: 16-lane group q reads contraction rows 32 ks + 8 q .. + 7,
// four at a time, lane s at row offset s / 4 and outer offset 4 (s % 4), as in frag_t_bf16.
template <int ROWS>
__device__ __forceinline__ bf16x8 frag_t16_bf16(const uint8_t* lds, int mbase, int ks, int lane) {
  const int q = lane >> 4, s = lane & 15;
  const int m = mbase + 4 * (s & 3);
  const int k = ks * 32 + 8 * q + (s >> 2);
  const int k2 = k + 4;
  const uint8_t* p0 = lds + k * (ROWS * 2) + (((m >> 3) ^ tr_swz(k)) << 4) + (m & 7) * 2;
  const uint8_t* p1 = lds + k2 * (ROWS * 2) + (((m >> 3) ^ tr_swz(k2)) << 4) + (m & 7) * 2;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)p1);
  typedef short i16x8 __attribute__((__vector_size__(8 * sizeof(short))));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

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

// LDS a tile needs beside its 128 KB of stages: the MXFP8 scale buffers.
constexpr int tile_sc_bytes(int fmt, int sched, int epi) {
  return fmt == F_MX ? (deep_pipe(fmt, sched, epi) ? 2 * 512 * 16 + 1024 : 2 * 512 * 16) : 32;
}

// Token-blocked MXFP8 of one 32-row block of two adjacent columns of an epilogue's bf16 output,
// read back from the staged tile: `rows` is the tile's fp32 staging (BN floats per row) whose
// slot(rl) float of row rl now holds the two bf16 values as one packed pair (low half: the first
// column). Each column gets the E8M0 exponent of its block's bf16 magnitude maximum and 32 E4M3
// codes (by the scaled conversion), exactly as the token-blocked quantizer makes them from the
// bf16 tensor for finite values; when ok, the codes go to q (first column) and q + ld_t
// (second), 32 contiguous bytes each. Returns the two E8M0 bytes (first column's in bits 0-7,
// second's in bits 8-15).
template <int BN, class Slot>
__device__ __forceinline__ uint32_t mx_colT_block(const float* rows, int rl0, const Slot& slot, uint8_t* q,
                                                  int64_t ld_t, bool ok) {
  uint32_t v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = __builtin_bit_cast(uint32_t, rows[(rl0 + r) * BN + slot(rl0 + r)]);
  uint32_t m = 0;                                        // both columns' magnitude maxima
#pragma unroll
  for (int r = 0; r < 32; ++r) m = pk_absmax_bits(m, v[r]);
  const int xlo = mx_exponent(m & 0xFFFFu), xhi = mx_exponent(m >> 16);
  const uint32_t bound = mx_bound_bits(xlo) | (mx_bound_bits(xhi) << 16);
  const float slo = mx_scale_operand(xlo), shi = mx_scale_operand(xhi);
  v4i qlo[2], qhi[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) {                          // rows 4k .. 4k + 3
    const uint32_t c0 = clamp_pair(v[4 * k], bound), c1 = clamp_pair(v[4 * k + 1], bound);
    const uint32_t c2 = clamp_pair(v[4 * k + 2], bound), c3 = clamp_pair(v[4 * k + 3], bound);
    // each column's two rows side by side: low halves, then high halves
    qlo[k >> 2][k & 3] = (int)e4m3x4_scaled(__builtin_amdgcn_perm(c1, c0, 0x05040100u),
                                            __builtin_amdgcn_perm(c3, c2, 0x05040100u), slo);
    qhi[k >> 2][k & 3] = (int)e4m3x4_scaled(__builtin_amdgcn_perm(c1, c0, 0x07060302u),
                                            __builtin_amdgcn_perm(c3, c2, 0x07060302u), shi);
  }
  if (ok) {
    reinterpret_cast<v4i*>(q)[0] = qlo[0];
    reinterpret_cast<v4i*>(q)[1] = qlo[1];
    reinterpret_cast<v4i*>(q + ld_t)[0] = qhi[0];
    reinterpret_cast<v4i*>(q + ld_t)[1] = qhi[1];
  }
  return (uint32_t)(xlo + 127) | ((uint32_t)(xhi + 127) << 8);
}

// The token-blocked output of one pass for a thread: two adjacent output columns whose bf16
// pairs overwrote float dw of the staged granule that sits at slot gran ^ (rl % 16) of each row
// rl, blocks k0 .. k0 + NB - 1 of the pass's four (rows 32 k .. + 31; rows 64+ in half1). feat
// is the first column's index in the token-blocked arrays, pos the pass's first position.
template <int BN, int NB>
__device__ __forceinline__ void mx_colT_run(const uint8_t* half0, const uint8_t* half1, int gran, int dw, int k0,
                                            uint8_t* qt, uint8_t* st, int64_t ld_t, int64_t feat, int64_t pos, bool ok) {
  auto slot = [&](int rl) { return ((gran ^ (rl & 15)) << 2) | dw; };
  uint32_t elo = 0, ehi = 0;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int k = k0 + b;
    const uint32_t e = mx_colT_block<BN>(reinterpret_cast<const float*>(k >= 2 ? half1 : half0), 32 * (k & 1), slot,
                                         qt + feat * ld_t + pos + 32 * k, ld_t, ok);
    elo |= (e & 0xFFu) << (8 * b);
    ehi |= (e >> 8) << (8 * b);
  }
  if (ok) {
    uint8_t* s = st + feat * (ld_t / 32) + (pos >> 5) + k0;
    if constexpr (NB == 4) {
      *reinterpret_cast<uint32_t*>(s) = elo;
      *reinterpret_cast<uint32_t*>(s + ld_t / 32) = ehi;
    } else if constexpr (NB == 2) {
      *reinterpret_cast<uint16_t*>(s) = (uint16_t)elo;
      *reinterpret_cast<uint16_t*>(s + ld_t / 32) = (uint16_t)ehi;
    } else {
      static_assert(NB == 1, "one, two or four blocks");
      s[0] = (uint8_t)elo;
      s[ld_t / 32] = (uint8_t)ehi;
    }
  }
}

// One output tile of one GEMM: tile number blk of the launch's tiles of this GEMM (a workgroup
// with blk % 8 == x runs on XCD x). lds_ (128 KB), sc_ (tile_sc_bytes) and amax_slot_ are the
// workgroup's LDS, which tiles of different GEMMs in one launch share.
template <int FMT, bool AK, bool BK, int EPI, int SCHED, int WGM, int WGN, int WMF, int WNF>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, int blk, uint8_t* lds_, uint8_t* sc_,
                                          uint32_t* amax_slot_) {
  constexpr int NWAVES = WGM * WGN;
  constexpr bool kMX = FMT == F_MX || FMT == F_MXU;
  constexpr int ES = FMT == F_BF16 ? 2 : 1;
  constexpr int WM = 32 * WMF, WN = 32 * WNF;
  constexpr int BM = WGM * WM, BN = WGN * WN;
  constexpr bool kDeep = deep_pipe(FMT, SCHED, EPI);
  constexpr int RB = kDeep ? 64 : kRowBytes;             // contraction bytes per LDS row and k-tile
  constexpr int NST = kDeep ? 4 : 2;                     // LDS stages
  constexpr int KT_ELEMS = RB / ES;                      // contraction elements per k-tile
  constexpr int A_BYTES = BM * RB, B_BYTES = BN * RB, STAGE = A_BYTES + B_BYTES;
  static_assert(NST * STAGE == 131072, "the stages fill the 128 KB the epilogue stages its tile through");
  uint8_t* const lds = lds_;
  // The epilogue stages fp32 rows through the two 64 KB halves of the same memory.
  uint8_t* const half0 = lds;
  uint8_t* const half1 = lds + NST * STAGE / 2;
  // MXFP8: E8M0 scales of 16 blocks of 32 per operand row (4 k-tiles of 128 bytes or 8 of 64),
  // double-buffered.
  constexpr int kScaleTiles = 512 / RB;
  constexpr int SC_BYTES = (FMT == F_MX && !kDeep) ? (BM + BN) * 4 * kScaleTiles : 16;
  static_assert(2 * SC_BYTES <= tile_sc_bytes(FMT, SCHED, EPI), "scale buffers");
  uint8_t (*const sc_lds)[SC_BYTES] = reinterpret_cast<uint8_t (*)[SC_BYTES]>(sc_);
  uint32_t& amax_slot = *amax_slot_;                     // FP8 (d)SwiGLU epilogues: the tile's amax

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  // ---------------------------------------------------------------- schedule
  int64_t m0, n0, row_end, k_begin = 0, k_end = p.K;
  const uint8_t* bptr = p.b;
  const uint8_t* bmx = p.b_mx;                           // MXFP8: E8M0 scales of B (this group's)
  uint16_t* cptr = p.c;
  int nt;
  int grp = 0;                                           // the group (E4M3 per-group scales)
  int64_t grp_lo = 0;                                    // row-partitioned: the group's first row
  if constexpr (SCHED == S_DENSE) {
    const int MT = p.mt_count, NT = p.nt_count;
    if (blk >= MT * NT) return;
    const int bid = xcd_tile(blk, MT * NT);
    const int GM = FMT == F_E4M3 ? 8 : SGE_XCD_GROUP_M;   // E4M3: 8 measured 1.2% faster (FP8 step)
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
    // Row tiles of all groups, counted from the clamped offsets; the grid is an upper bound.
    int total = 0;
    {
      int64_t prev = 0;
      for (int gg = 0; gg < p.G; ++gg) {
        int64_t a = p.offsets[gg], b = p.offsets[gg + 1];
        a = a < prev ? prev : (a > p.T ? p.T : a);
        b = b < a ? a : (b > p.T ? p.T : b);
        prev = b;
        total += (int)((b - a + BM - 1) / BM);
      }
    }
    total *= p.nt_count;
    if (blk >= total) return;                            // beyond the last real tile
    // Each group's row tiles x column tiles are contiguous in t; inside a group they go in
    // bands of SGE_GROUPED_GM row tiles, row tile fastest, so the tiles an XCD runs together
    // share a few panels of both operands (a 16-column-tile gated fc1 otherwise spans 2 row
    // bands x 16 weight panels per 32 tiles).
    int w = xcd_tile(blk, total);
    int g = -1, mtg = 0;
    int64_t lo = 0, hi = 0, prev = 0;
    for (int gg = 0; gg < p.G; ++gg) {
      int64_t a = p.offsets[gg], b = p.offsets[gg + 1];
      a = a < prev ? prev : (a > p.T ? p.T : a);
      b = b < a ? a : (b > p.T ? p.T : b);
      prev = b;
      const int tiles = (int)((b - a + BM - 1) / BM);
      if (w < tiles * p.nt_count) { g = gg; lo = a; hi = b; mtg = tiles; break; }
      w -= tiles * p.nt_count;
    }
    if (g < 0) return;                                   // beyond the last real tile
    // Bands of 8 for plain stores with a K-major weight (4-10% faster fc2 forward and FP8 /
    // MXFP8 fc1 dgrad than 4), 4 elsewhere (8 is 4-6% slower on the gated fc1 forward and
    // the bf16 dgrad, whose weight is read N-major).
    constexpr int GMG = (EPI == E_STORE && BK) ? SGE_GROUPED_GM_STORE : SGE_GROUPED_GM;
    const int first = w / (GMG * p.nt_count) * GMG;
    const int gsz = min(mtg - first, GMG);
    const int in_band = w % (GMG * p.nt_count);
    const int lin = first + in_band % gsz;
    nt = in_band / gsz;
    grp = g;
    grp_lo = lo;
    m0 = lo + (int64_t)lin * BM;
    row_end = hi;
    n0 = (int64_t)nt * (glu_fwd(EPI) ? BN / 2 : BN);
    bptr += (int64_t)g * p.b_group_stride * ES;
    if constexpr (FMT == F_MX || FMT == F_MXU) bmx += (int64_t)g * p.b_mx_group_stride;
  } else {
    // Groups differ in length (their contraction), so every XCD takes an equal contiguous
    // slice of each group's tiles: balanced XCDs, and an XCD's concurrent tiles still share
    // panels. (Identity when the tiles of a group do not split evenly over 8 XCDs.)
    const int per = p.mt_count * p.nt_count;
    if (blk >= per * p.G) return;
    int t = blk;
    if ((per & 7) == 0) {
      const int per8 = per >> 3, x = t & 7, i = t >> 3;
      t = (i / per8) * per + x * per8 + i % per8;
    }
    const int g = t / per;
    grp = g;
    const int rem = t % per;
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
  const int64_t n_end = glu_fwd(EPI) ? p.F : p.N;

  // ---------------------------------------------------------------- main loop
  // bf16 (kM16): each 32x32 block (i, j) of the wave's output is four 16x16x32 MFMA tiles
  // acc4[i][j][2 ii + jj] (rows 16 ii.., columns 16 jj..); under the power limit that holds the
  // clock down under MFMA load, register-only 16x16x32 loops sustain ~13% more bf16 FLOP/s
  // than 32x32x16 ones on MI355X. 8-bit formats: one 32x32 accumulator per block.
  constexpr bool kM16 = FMT == F_BF16 && SGE_BF16_M16;
  f32x16 acc[WMF][WNF];
  f32x4 acc4[WMF][WNF][4];
#pragma unroll
  for (int i = 0; i < WMF; ++i)
#pragma unroll
    for (int j = 0; j < WNF; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (kM16) acc4[i][j][e >> 2][e & 3] = 0.0f;
        else acc[i][j][e] = 0.0f;
      }
    }

  IdentityRows idrows;
  SwigluRows<WN> swrows{p.F};
  // Rows of B: N (dense / group M, 2F for SwiGLU), or the N_out rows of group K.
  const int64_t b_rows = glu_fwd(EPI) ? 2 * p.F : p.N;

  // Tile copies. Inner-contiguous operands are addressed from their first tile row,
  // outer-contiguous ones from the tile's first outer column of contraction row 0.
  TileCopy<BM, AK, ES, NWAVES, RB> ca;
  TileCopy<BN, BK, ES, NWAVES, RB> cb;
  const uint8_t* a_base = AK ? p.a + m0 * p.lda * ES : p.a + m0 * 2;
  const int64_t a_bytes = AK ? ((SCHED == S_GROUP_M ? p.T : p.M) - m0) * p.lda * ES : p.K * p.lda * 2 - m0 * 2;
  const uint8_t* b_base = BK ? bptr + n0 * p.ldb * ES : bptr + n0 * 2;
  const int64_t b_bytes = BK ? (b_rows - n0) * p.ldb * ES : p.K * p.ldb * 2 - n0 * 2;
  ca.init(p.lda, m0, row_end, idrows);
  if constexpr (glu_fwd(EPI)) cb.init(p.ldb, n0, b_rows, swrows);
  else cb.init(p.ldb, n0, b_rows, idrows);

  auto issue_tile = [&](uint8_t* buf, int64_t k0) {
    ca.issue(buf, a_base, p.lda, a_bytes, k0, k_end);
    cb.issue(buf + A_BYTES, b_base, p.ldb, b_bytes, k0, k_end);
  };

  // MX scales: one dword per fragment row holds the 4 E8M0 bytes of a k-tile,
  // pre-shifted so byte 2*ks of the register is this lane's 32-block. When the scale
  // rows are dword-aligned, 16 bytes per row (4 k-tiles) move to LDS by DMA and each
  // k-tile reads its dword from there; otherwise bytes are read from global memory.
  uint32_t sa[WMF], sb[WNF], san[WMF], sbn[WNF];
  constexpr bool mx_lds = FMT == F_MX;
  auto issue_scales = [&](int group, int buf) {
    if constexpr (FMT == F_MX) {
      // 1-KB pieces: 64 rows x 16 bytes; A rows then B rows.
      constexpr int kPieces = (BM + BN) / 64;
      const int64_t blk0 = (k_begin >> 5) + (int64_t)group * 16;
      const int64_t nblk = (k_end + 31) >> 5;
#pragma unroll
      for (int it = 0; it < (kPieces + NWAVES - 1) / NWAVES; ++it) {
        const int piece = it * NWAVES + wave;
        if (piece >= kPieces) break;
        const bool is_a = piece < BM / 64;
        const int r = (is_a ? piece : piece - BM / 64) * 64 + lane;
        // B rows follow the tile's row map (the SwiGLU gate/up interleave)
        const int64_t row = is_a ? m0 + r : (glu_fwd(EPI) ? swrows(n0, r) : n0 + r);
        const bool ok = row < (is_a ? row_end : b_rows) && blk0 < nblk;
        const uint8_t* base = is_a ? p.a_mx : bmx;
        const int64_t ld = is_a ? p.a_mx_ld : p.b_mx_ld;
        const int64_t rows_total = is_a ? (SCHED == S_GROUP_M ? p.T : p.M) : b_rows;
        // B's scales of one group can sit inside wider rows (b_mx_bytes: the whole array), so the
        // resource ends where the array ends, not rows_total rows after this group's start.
        const int64_t avail = (!is_a && p.b_mx_bytes) ? (int64_t)((p.b_mx + p.b_mx_bytes) - (bmx + blk0))
                                                      : rows_total * ld - blk0;
        const i32x4 rs = make_rsrc4(base + blk0, avail);
        lds_copy16(rs, sc_lds[buf] + piece * 1024, ok ? (uint32_t)(row * ld) : kOOB);
      }
    }
  };
  auto load_scales = [&](int64_t k0, uint32_t (&da)[WMF], uint32_t (&db)[WNF]) {
    if constexpr (kMX) {
      const int sh = 8 * (lane >> 5);
      if constexpr (mx_lds) {
        const int t = (int)((k0 - k_begin) / KT_ELEMS);
        // a k-tile's RB/32 bytes start at byte (t % kScaleTiles) * RB/32 of the row's 16; 64-byte
        // tiles take the aligned dword holding their 2 bytes and shift the odd tile's down
        const int byte0 = (t % kScaleTiles) * (RB / 32);
        const uint8_t* sl = sc_lds[(t / kScaleTiles) & 1] + (byte0 & ~3);
        const int sh2 = sh + 8 * (byte0 & 3);
#pragma unroll
        for (int i = 0; i < WMF; ++i)
          da[i] = *reinterpret_cast<const uint32_t*>(sl + (wm * WM + i * 32 + (lane & 31)) * 16) >> sh2;
#pragma unroll
        for (int j = 0; j < WNF; ++j)
          db[j] = *reinterpret_cast<const uint32_t*>(sl + (BM + wn * WN + j * 32 + (lane & 31)) * 16) >> sh2;
        return;
      }
      const int64_t blk0 = k0 >> 5;
      const int64_t nblk = (k_end + 31) >> 5;
#pragma unroll
      for (int i = 0; i < WMF; ++i) {
        const int64_t row = m0 + wm * WM + i * 32 + (lane & 31);
        uint32_t v = 0x7F7F7F7Fu;
        if (row < row_end) {
          const uint8_t* s = p.a_mx + row * p.a_mx_ld + blk0;
          v = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) v |= (blk0 + e < nblk ? (uint32_t)s[e] : 127u) << (8 * e);
        }
        da[i] = v >> sh;
      }
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        const int rr = wn * WN + j * 32 + (lane & 31);
        const int64_t row = glu_fwd(EPI) ? swrows(n0, rr) : n0 + rr;
        uint32_t v = 0x7F7F7F7Fu;
        if (row < b_rows) {
          const uint8_t* s = bmx + row * p.b_mx_ld + blk0;
          v = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) v |= (blk0 + e < nblk ? (uint32_t)s[e] : 127u) << (8 * e);
        }
        db[j] = v >> sh;
      }
    }
  };

  const int64_t klen = k_end - k_begin;
  const int KT = klen > 0 ? (int)((klen + KT_ELEMS - 1) / KT_ELEMS) : 0;
  const int lrow = lane & 31;
  const int lhalf = lane >> 5;

  // Fragments: 8 bf16 (32x32x16) or 32 fp8 (32x32x64) contraction values per lane.
  using Frag = typename std::conditional<FMT == F_BF16, bf16x8, i32x8>::type;
  constexpr int KS = FMT == F_BF16 ? RB / 32 : RB / 64;             // MFMA k-steps per tile
  constexpr int kReads = FMT == F_BF16 ? (AK ? WMF : 2 * WMF) + (BK ? WNF : 2 * WNF) : 2 * (WMF + WNF);
  constexpr int kMfma = WMF * WNF;

  auto rd = [&](const uint8_t* buf, int ks, Frag (&fa)[WMF], Frag (&fb)[WNF]) {
    const uint8_t* a_lds = buf;
    const uint8_t* b_lds = buf + A_BYTES;
    // Reads go out in the order the MFMAs consume them: A0, B0..B(WNF-1), A1, A2, ...
    if constexpr (FMT == F_BF16) {
      auto ra = [&](int i) {
        fa[i] = AK ? frag_k_bf16(a_lds, wm * WM + i * 32 + lrow, ks * 2 + lhalf)
                   : frag_t_bf16<BM>(a_lds, wm * WM + i * 32, ks, lane);
      };
      ra(0);
#pragma unroll
      for (int j = 0; j < WNF; ++j)
        fb[j] = BK ? frag_k_bf16(b_lds, wn * WN + j * 32 + lrow, ks * 2 + lhalf)
                   : frag_t_bf16<BN>(b_lds, wn * WN + j * 32, ks, lane);
#pragma unroll
      for (int i = 1; i < WMF; ++i) ra(i);
    } else {
      // f8f6f4 32x32x64 lane layout: bytes 0-15 hold k = 16*half .. +15 and
      // bytes 16-31 hold k = 32 + 16*half .. +15 of the 64-wide step.
      auto rd8 = [&](const uint8_t* base, int r) {
        const int c0 = ks * 4 + lhalf, c1 = c0 + 2;
        const uint8_t* row = base + r * RB;
        const int4 lo = *reinterpret_cast<const int4*>(row + ((c0 ^ swz_rows<RB>(r)) << 4));
        const int4 hi = *reinterpret_cast<const int4*>(row + ((c1 ^ swz_rows<RB>(r)) << 4));
        return i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      fa[0] = rd8(a_lds, wm * WM + lrow);
#pragma unroll
      for (int j = 0; j < WNF; ++j) fb[j] = rd8(b_lds, wn * WN + j * 32 + lrow);
#pragma unroll
      for (int i = 1; i < WMF; ++i) fa[i] = rd8(a_lds, wm * WM + i * 32 + lrow);
    }
  };

  auto mma = [&](int ks, const Frag (&fa)[WMF], const Frag (&fb)[WNF]) {
#pragma unroll
    for (int i = 0; i < WMF; ++i)
#pragma unroll
      for (int j = 0; j < WNF; ++j) {
        if constexpr (FMT == F_BF16) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
        } else if constexpr (kMX) {
          // byte 2*ks of the pre-shifted scale registers is this lane's 32-block
          if (ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0,
                                                                        (int)sb[j], 0, (int)sa[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 2,
                                                                        (int)sb[j], 2, (int)sa[i]);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, 0, 0, 0x7F7F7F7F,
                                                                      0, 0x7F7F7F7F);
        }
      }
  };

  // Issue order inside a scheduling region: the next step's fragment reads go out early,
  // kRdPer after each of the first MFMAs, and the remaining MFMAs cover their latency.
  constexpr int kRdPer0 = kMX ? SGE_RD_PER_MFMA_MX : (SCHED != S_DENSE ? SGE_RD_PER_MFMA_GROUPED : SGE_RD_PER_MFMA);
  constexpr int kRdPer = kRdPer0 * kMfma >= kReads ? kRdPer0 : (kReads + kMfma - 1) / kMfma;
  constexpr int kRdFull = kReads / kRdPer, kRdRem = kReads % kRdPer;
  constexpr int kRdUsed = kRdFull + (kRdRem ? 1 : 0);
  auto interleave = [&](int steps) {
    for (int s = 0; s < steps; ++s) {
#pragma unroll
      for (int t = 0; t < kRdFull; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kRdPer, 0);
      }
      if constexpr (kRdRem > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kRdRem, 0);
      }
      if constexpr (kMfma > kRdUsed) __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kRdUsed, 0);
    }
  };

  Frag fa[2][WMF], fb[2][WNF];
  if constexpr (kDeep) {
    // NST k-tiles of copies are in flight: the fragments of a tile (one MFMA k-step) are all in
    // registers before its MFMAs run, so once every wave has passed the barrier that follows
    // those reads, the tile's stage is refilled with the tile NST ahead. Each tile's barrier
    // is preceded by the wave's wait for its own copies of the next tile (vector loads complete
    // in the order issued, so the copies of later tiles stay in flight) and for its own LDS
    // reads; after it, that next tile's stage is visible to every wave.
    // MXFP8 scales: the 16 E8M0 bytes of 8 k-tiles per operand row (one 16-byte piece of the row,
    // as whole lines are fetched) go to one of two LDS buffers while the 8 tiles before them are
    // multiplied. Every tile issues that copy (so each tile has the same count of copies to wait
    // for); on the 7 tiles of 8 that are not due, its lanes take an out-of-range offset, which
    // reads nothing from memory, and it lands in a dummy LDS area.
    // A steady-state tile is one basic block with an explicit order: two MFMAs, the wait and
    // the barrier, then each remaining MFMA followed by one copy of the tile NST ahead and one
    // fragment (with its scale) of the next tile. Fragments and scales are double-buffered by
    // tile parity (the loop body is written out twice so every register index is a constant).
    static_assert(FMT != F_BF16 && KS == 1 && NST == 4, "deep pipeline: 8-bit, one k-step per k-tile");
    constexpr int kMT = KS * kMfma;                     // MFMAs per tile
    constexpr int kFPS = WMF + WNF;                     // fragments per k-step: A0, B0.., A1..
    constexpr int kFT = KS * kFPS;                      // fragments per tile
    constexpr int kGrpTiles = 8;                        // k-tiles per scale group (16 blocks of 32)
    static_assert(!kMX || NST == 4, "the scale groups are timed for four stages");
    constexpr int SC_GROUP = kMX ? (BM + BN) * 16 : 0;  // scale bytes per group
    constexpr int kScPer = SC_GROUP / 1024 / NWAVES;    // 1-KB pieces (64 rows) per wave
    static_assert(!kMX || kScPer * 1024 * NWAVES == SC_GROUP, "scale pieces split evenly over the waves");
    constexpr int kCa = decltype(ca)::kInstr, kCb = decltype(cb)::kInstr;
    constexpr int CPT = kCa + kCb + kScPer;             // copies per tile per wave
    constexpr int kHead = 2;                            // MFMAs issued before the wait and the barrier
    static_assert(CPT <= kMT - kHead && kFT <= kMT - kHead, "one copy and one fragment after each MFMA");
    // two group buffers, then the dummy area the off-cycle copies land in
    static_assert(!kMX || 2 * SC_GROUP + 1024 <= tile_sc_bytes(FMT, SCHED, EPI), "scale buffers");
    uint8_t* const sc_st = sc_;
    uint32_t sa2[2][WMF], sb2[2][WNF];
    Frag fa2[2][KS][WMF], fb2[2][KS][WNF];              // [tile parity][k-step][fragment]
    auto stage = [&](int t) { return lds + (t % NST) * STAGE; };
    uint32_t sc_off[kMX ? kScPer : 1];
    bool sc_isa[kMX ? kScPer : 1];
    if constexpr (kMX) {
#pragma unroll
      for (int it = 0; it < kScPer; ++it) {
        const int piece = it * NWAVES + wave;
        const bool is_a = piece < BM / 64;
        const int r = (is_a ? piece : piece - BM / 64) * 64 + lane;
        // B rows follow the tile's row map (the gate / up interleave of a gated fc1)
        const int64_t row = is_a ? m0 + r : (glu_fwd(EPI) ? swrows(n0, r) : n0 + r);
        const bool ok = row < (is_a ? row_end : b_rows);
        sc_isa[it] = is_a;
        // the row's scale bytes from the first block of this tile run's contraction range
        sc_off[it] = ok ? (uint32_t)(row * (is_a ? p.a_mx_ld : p.b_mx_ld) + (k_begin >> 5)) : kOOB;
      }
    }
    // A's scales: rows of the whole operand; B's: to the end of the scale array (one expert's
    // rows can sit inside wider rows holding every expert's)
    const int64_t a_rows_total = SCHED == S_GROUP_M ? p.T : p.M;
    const i32x4 rs_a = make_rsrc4(p.a_mx, kMX ? a_rows_total * p.a_mx_ld : 0);
    const i32x4 rs_b = make_rsrc4(bmx, !kMX ? 0 : (p.b_mx_bytes ? (int64_t)((p.b_mx + p.b_mx_bytes) - bmx)
                                                                 : b_rows * p.b_mx_ld));
    // Copy number c (0 .. CPT-1) made while tile t - NST is multiplied: the A and B pieces of tile
    // t, then, when t % 8 == 4, the scale pieces of group g = t / 8 + 1. That group is first
    // read at tile t + 4 (whose copies follow these); its buffer held group g - 2, last read at
    // tile t - 5, before the barrier of the tile being multiplied.
    auto copy = [&](int t, int c) {
      const int64_t k0 = k_begin + (int64_t)t * KT_ELEMS;
      uint8_t* buf = stage(t);
      if (c < kCa) {
        // resources based at the tile's first contraction element keep the offsets 32-bit
        const int64_t sh = AK ? k0 * ES : k0 * p.lda * 2;
        const i32x4 rsrc = make_rsrc4(a_base + sh, a_bytes - sh);
        lds_copy16(rsrc, buf + (NWAVES * c + wave) * 1024, (k0 + ca.kk[c] < k_end) ? ca.off[c] : kOOB);
      } else if (c < kCa + kCb) {
        const int i = c - kCa;
        const int64_t sh = BK ? k0 * ES : k0 * p.ldb * 2;
        const i32x4 rsrc = make_rsrc4(b_base + sh, b_bytes - sh);
        lds_copy16(rsrc, buf + A_BYTES + (NWAVES * i + wave) * 1024, (k0 + cb.kk[i] < k_end) ? cb.off[i] : kOOB);
      } else if constexpr (kMX) {
        const int it = c - kCa - kCb;
        const int piece = it * NWAVES + wave;
        const int g = t / kGrpTiles + 1;
        const bool due = t % kGrpTiles == kGrpTiles / 2 && g * kGrpTiles < KT;
        const uint8_t* dst = due ? sc_st + (g & 1) * SC_GROUP + piece * 1024 : sc_st + 2 * SC_GROUP;
        const uint32_t o = (due && sc_off[it] != kOOB) ? sc_off[it] + (uint32_t)(g * 16) : kOOB;
        lds_copy16(sc_isa[it] ? rs_a : rs_b, dst, o);
      }
    };
    // Fragment f of tile t: A0, B0.., A1.. (the order the MFMAs use them): 32 bytes from two
    // 16-byte chunks of a 64-byte row. MXFP8: also the dword of the row's E8M0 bytes that holds
    // the blocks of tiles t and t + 1 for even t (the two lane halves read the same dword: a
    // broadcast, not a bank conflict); the even tile shifts it by 8 bits in the upper lane half,
    // the odd tile after it takes that shifted copy, and each selects byte 2 * (t % 2) in the MFMA.
    auto frag = [&](int t, int f, Frag (&fa_)[KS][WMF], Frag (&fb_)[KS][WNF], uint32_t (&sa_)[WMF],
                    uint32_t (&sb_)[WNF], auto odd_t) {
      const uint8_t* buf = stage(t);
      const int ks = f / kFPS, g = f % kFPS;
      const bool is_a = g == 0 || g > WNF;
      const int idx = g == 0 ? 0 : (g > WNF ? g - WNF : g - 1);
      const int rbase = is_a ? wm * WM + idx * 32 : wn * WN + idx * 32;
      const int r = rbase + lrow;
      const uint8_t* opl = buf + (is_a ? 0 : A_BYTES);
      const uint8_t* row = opl + r * RB;
      const int4 lo = *reinterpret_cast<const int4*>(row + ((lhalf ^ swz_rows<RB>(r)) << 4));
      const int4 hi = *reinterpret_cast<const int4*>(row + (((2 + lhalf) ^ swz_rows<RB>(r)) << 4));
      const Frag v = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (is_a) fa_[ks][idx] = v;
      else fb_[ks][idx] = v;
      if constexpr (kMX) {
        if constexpr (decltype(odd_t)::value) {
          // an odd tile's two blocks sit in the dword its even predecessor read (and shifted)
          if (is_a) sa_[idx] = sa2[0][idx];
          else sb_[idx] = sb2[0][idx];
        } else {
          const uint8_t* sl = sc_st + ((t / kGrpTiles) & 1) * SC_GROUP;
          const uint32_t e =
              *reinterpret_cast<const uint32_t*>(sl + ((is_a ? 0 : BM) + r) * 16 + 4 * ((t % kGrpTiles) >> 1));
          if (is_a) sa_[idx] = e;
          else sb_[idx] = e;
        }
      }
    };
    auto mma1 = [&](const Frag (&fa_)[KS][WMF], const Frag (&fb_)[KS][WNF], const uint32_t (&sa_)[WMF],
                    const uint32_t (&sb_)[WNF], int q, auto odd_c) {
      const int ks = q / kMfma, i = (q % kMfma) / WNF, j = q % WNF;
      constexpr int sel = 2 * decltype(odd_c)::value;   // byte of the tile's first block
      if constexpr (kMX)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb_[ks][j], fa_[ks][i], acc[i][j], 0, 0, sel,
                                                                    (int)sb_[j], sel, (int)sa_[i]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb_[ks][j], fa_[ks][i], acc[i][j], 0, 0, 0,
                                                                    0x7F7F7F7F, 0, 0x7F7F7F7F);
    };
    auto barrier_after = [&](auto n_c) {               // own copies down to n outstanding, then barrier
      constexpr int n = decltype(n_c)::value;
      if constexpr (n == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
    };
    // tile t landed; issued_after (0 .. NST-1): tiles issued after it
    auto wait_tile = [&](int t, int issued_after) {
      switch (issued_after < NST - 1 ? issued_after : NST - 1) {
        case 3: barrier_after(std::integral_constant<int, 3 * CPT>{}); break;
        case 2: barrier_after(std::integral_constant<int, 2 * CPT>{}); break;
        case 1: barrier_after(std::integral_constant<int, CPT>{}); break;
        default: barrier_after(std::integral_constant<int, 0>{}); break;
      }
    };
    if (KT > 0) {
      if constexpr (kMX) {                              // group 0's scales, before every tile copy
#pragma unroll
        for (int it = 0; it < kScPer; ++it) {
          const int piece = it * NWAVES + wave;
          lds_copy16(sc_isa[it] ? rs_a : rs_b, sc_st + piece * 1024, sc_off[it]);
        }
      }
#pragma unroll
      for (int t = 0; t < NST; ++t)
        if (t < KT)
#pragma unroll
          for (int c = 0; c < CPT; ++c) copy(t, c);
      wait_tile(0, KT - 1 < NST - 1 ? KT - 1 : NST - 1);
#pragma unroll
      for (int f = 0; f < kFT; ++f) frag(0, f, fa2[0], fb2[0], sa2[0], sb2[0], std::false_type{});
    }
    // Tile kt (parity P): tile kt + NST exists (steady) or not (tail).
    auto tile = [&](int kt, auto par, auto steady_c) {
      constexpr int P = decltype(par)::value, Q = P ^ 1;
      constexpr bool steady = decltype(steady_c)::value;
      const std::integral_constant<int, P> odd{};        // tile kt is odd exactly when P == 1
      if constexpr (kMX && P == 0) {                     // the upper lane half's block is the next byte
#pragma unroll                                           // (odd tiles copy the shifted dword)
        for (int i = 0; i < WMF; ++i) sa2[P][i] >>= 8 * lhalf;
#pragma unroll
        for (int j = 0; j < WNF; ++j) sb2[P][j] >>= 8 * lhalf;
      }
#pragma unroll
      for (int q = 0; q < kHead; ++q) mma1(fa2[P], fb2[P], sa2[P], sb2[P], q, odd);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (steady) {
        barrier_after(std::integral_constant<int, (NST - 2) * CPT>{});   // tiles kt+2 .. kt+NST-1 stay in flight
      } else {
        if (kt + 1 < KT) wait_tile(kt + 1, KT - 2 - kt < NST - 2 ? KT - 2 - kt : NST - 2);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = kHead; q < kMT; ++q) {
        mma1(fa2[P], fb2[P], sa2[P], sb2[P], q, odd);
        const int s_ = q - kHead;
        if constexpr (steady) {
          if (s_ < CPT) copy(kt + NST, s_);
          if (s_ < kFT) frag(kt + 1, s_, fa2[Q], fb2[Q], sa2[Q], sb2[Q], std::integral_constant<bool, Q == 1>{});
        } else {
          if (s_ < CPT && kt + NST < KT) copy(kt + NST, s_);
          if (s_ < kFT && kt + 1 < KT) frag(kt + 1, s_, fa2[Q], fb2[Q], sa2[Q], sb2[Q], std::integral_constant<bool, Q == 1>{});
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using S1 = std::integral_constant<bool, true>;
    using S0 = std::integral_constant<bool, false>;
    int kt = 0;
    for (; kt + 1 + NST < KT; kt += 2) {                // tiles kt + NST and kt + 1 + NST exist
      tile(kt, std::integral_constant<int, 0>{}, S1{});
      tile(kt + 1, std::integral_constant<int, 1>{}, S1{});
    }
    for (; kt < KT; kt += 2) {                          // at most NST + 1 tiles
      tile(kt, std::integral_constant<int, 0>{}, S0{});
      if (kt + 1 < KT) tile(kt + 1, std::integral_constant<int, 1>{}, S0{});
    }
  } else if constexpr (kM16) {
    // bf16 on 16x16x32 MFMAs, two LDS stages of 64-element k-tiles (two MFMA k-steps each).
    // Fragments: the wave's 2 WMF A pieces of 16 rows and 2 WNF B pieces. A pieces are read in
    // place (piece f of the next step goes into fa16[f] right after the last MFMA that used it),
    // except the last one, which is double-buffered by step parity so that the step's last
    // fragment read is not the last instruction before the next step's first MFMAs; B pieces are
    // double-buffered. The barrier of tile kt sits after the first MFMAs of its second step,
    // behind each wave's wait for its copies of tile kt + 1; after it the copies of tile kt + 2
    // go into tile kt's stage (every wave has its fragments of that stage in registers),
    // SGE_M16_CPG after each group of MFMAs from the first on, so a copy has nearly a whole tile
    // of MFMAs to land.
    constexpr int FA = 2 * WMF, FB = 2 * WNF;
    constexpr int CPT = decltype(ca)::kInstr + decltype(cb)::kInstr;   // copies per tile per wave
    static_assert(CPT <= FA * SGE_M16_CPG, "copies fit the groups");
    static_assert(FB < FA - 1, "B reads before the last A read");
    bf16x8 fa16[FA - 1], fa16l[2], fb16[2][FB];
    auto rd_a = [&](const uint8_t* buf, int ks, int f, bf16x8& dst) {
      const int mb = wm * WM + f * 16;
      dst = AK ? frag_k16_bf16(buf, mb, ks, lane) : frag_t16_bf16<BM>(buf, mb, ks, lane);
    };
    auto rd_b = [&](const uint8_t* buf, int ks, int f, bf16x8 (&fb)[FB]) {
      const int nb = wn * WN + f * 16;
      const uint8_t* b_lds = buf + A_BYTES;
      fb[f] = BK ? frag_k16_bf16(b_lds, nb, ks, lane) : frag_t16_bf16<BN>(b_lds, nb, ks, lane);
    };
    // The copies of one tile: buffer resources based at its first contraction element (32-bit
    // offsets), its LDS stage, and its contraction extent (chunks at or past it read zeros).
    struct TileSrc {
      i32x4 ra, rb;
      uint32_t dst;
      int klim;
    };
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = lds_addr_of(lds);
    auto tile_src = [&](int t) {
      const int64_t k0 = k_begin + (int64_t)t * KT_ELEMS;
      const int64_t sa = AK ? k0 * 2 : k0 * p.lda * 2, sb = BK ? k0 * 2 : k0 * p.ldb * 2;
      const int64_t kl = k_end - k0;
      return TileSrc{make_rsrc4(a_base + sa, a_bytes - sa), make_rsrc4(b_base + sb, b_bytes - sb),
                     lds0 + (uint32_t)((t & 1) * STAGE), (int)(kl < KT_ELEMS ? kl : KT_ELEMS)};
    };
    // Copy c (0 .. CPT-1) of a tile: A's pieces, then B's.
    auto copy1 = [&](const TileSrc& ts, int c) {
      if (c < decltype(ca)::kInstr) {
        lds_copy16_at(ts.ra, ts.dst + (uint32_t)((NWAVES * c + wave_s) * 1024), ca.kk[c] < ts.klim ? ca.off[c] : kOOB);
      } else {
        const int i = c - decltype(ca)::kInstr;
        lds_copy16_at(ts.rb, ts.dst + (uint32_t)(A_BYTES + (NWAVES * i + wave_s) * 1024),
                      cb.kk[i] < ts.klim ? cb.off[i] : kOOB);
      }
    };
    // One k-step of parity P on (fa16, fa16l[P], fbc): for each A piece f its 2 WNF MFMAs, then
    // its read for the step (nbuf, nks), the last piece's into fa16l[P ^ 1] with piece FB's; B
    // reads into fbn over the first FB groups. A tile's second step (P == 1) puts the wait for
    // the next tile's copies and the barrier after its first group, and with COPY (and do_copy)
    // issues SGE_M16_CPG copies of the tile ts after each group.
    auto step = [&](auto par, auto copy_c, const bf16x8 (&fbc)[FB], bf16x8 (&fbn)[FB], const uint8_t* nbuf, int nks,
                    const TileSrc& ts, bool do_copy) {
      constexpr int P = decltype(par)::value;
      constexpr bool COPY = decltype(copy_c)::value;
      auto group = [&](int f, const bf16x8& a) {
        const int i = f >> 1, ii = f & 1;
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            acc4[i][j][2 * ii + jj] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(fbc[2 * j + jj], a, acc4[i][j][2 * ii + jj], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (P == 1 && f == 0) {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");             // the next tile landed
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");           // this wave's reads of its stage done
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto after = [&](int f) {                          // B read and copy of group f
        if (f < FB) rd_b(nbuf, nks, f, fbn);
        if constexpr (COPY) {
#pragma unroll
          for (int u = 0; u < SGE_M16_CPG; ++u)
            if (f * SGE_M16_CPG + u < CPT && do_copy) copy1(ts, f * SGE_M16_CPG + u);
        }
        __builtin_amdgcn_sched_barrier(0);
      };
#pragma unroll
      for (int f = 0; f < FA - 1; ++f) {
        group(f, fa16[f]);
        rd_a(nbuf, nks, f, fa16[f]);
        if (f == FB) rd_a(nbuf, nks, FA - 1, fa16l[P ^ 1]);
        after(f);
      }
      group(FA - 1, fa16l[P]);
      after(FA - 1);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using C0 = std::false_type;
    using C1 = std::true_type;
    if (KT > 0) {
      issue_tile(lds, k_begin);
      if (KT > 1) {
        issue_tile(lds + STAGE, k_begin + KT_ELEMS);
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPT) : "memory");   // tile 0 landed, tile 1 in flight
      } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      }
      __syncthreads();
#pragma unroll
      for (int f = 0; f < FA - 1; ++f) {
        rd_a(lds, 0, f, fa16[f]);
        if (f < FB) rd_b(lds, 0, f, fb16[0]);
      }
      rd_a(lds, 0, FA - 1, fa16l[0]);
    }
    for (int kt = 0; kt < KT; ++kt) {
      uint8_t* const cur = (kt & 1) ? lds + STAGE : lds;
      const uint8_t* const nxt = (kt & 1) ? lds : lds + STAGE;
      const TileSrc ts = tile_src(kt + 2);                            // into stage kt % 2
      step(I0{}, C0{}, fb16[0], fb16[1], cur, 1, ts, false);
      // On the last tile the second step reads a stale stage: in bounds, never used.
      step(I1{}, C1{}, fb16[1], fb16[0], nxt, 0, ts, kt + 2 < KT);
    }
  } else {
  // Each wave waits for its own direct-to-LDS copies, then the barrier makes the
  // whole stage visible (and frees the other stage for the next copies).
  auto stage_done = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  // Software pipeline: fragments of k-step s+1 are read while the MFMAs of step s
  // run; the barrier sits before the tile's last k-step, whose MFMAs cover the
  // reads of the next tile's first fragments (the fragments of that last step
  // are already in registers, so the other stage may be refilled).
  uint8_t* const st0 = lds;
  uint8_t* const st1 = lds + STAGE;
  if (KT > 0) {
    issue_tile(st0, k_begin);
    if constexpr (mx_lds) issue_scales(0, 0);
    stage_done();
    load_scales(k_begin, sa, sb);
    rd(st0, 0, fa[0], fb[0]);
  }
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* cur = (kt & 1) ? st1 : st0;
    uint8_t* nxt = (kt & 1) ? st0 : st1;
    if (kt + 1 < KT) {
      issue_tile(nxt, k_begin + (int64_t)(kt + 1) * KT_ELEMS);
      if constexpr (kMX && !mx_lds) load_scales(k_begin + (int64_t)(kt + 1) * KT_ELEMS, san, sbn);
    }
    // Scales of the next group of k-tiles: the buffer they fill was last read before the
    // previous barrier; they land at least one barrier before use.
    if constexpr (mx_lds) {
      if (kt % kScaleTiles == 0 && (kt / kScaleTiles + 1) * kScaleTiles < KT)
        issue_scales(kt / kScaleTiles + 1, (kt / kScaleTiles + 1) & 1);
    }
    __builtin_amdgcn_sched_barrier(0);   // the copies leave first: their latency spans the tile
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      rd(cur, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mma(ks, fa[ks & 1], fb[ks & 1]);
    }
    interleave(KS - 1);
    stage_done();
    // On the last tile this reads a stale stage: in bounds, never used.
    rd(nxt, 0, fa[0], fb[0]);
    mma(KS - 1, fa[1], fb[1]);
    interleave(1);
    if constexpr (kMX) {
      if constexpr (mx_lds) {
        load_scales(k_begin + (int64_t)(kt + 1) * KT_ELEMS, sa, sb);
      } else {
#pragma unroll
        for (int i = 0; i < WMF; ++i) sa[i] = san[i];
#pragma unroll
        for (int j = 0; j < WNF; ++j) sb[j] = sbn[j];
      }
    }
  }
  }

  // ---------------------------------------------------------------- epilogue
  // Branch-free: every global access is a buffer op over the output tile whose
  // out-of-range lanes read zeros / drop their writes, so all loads of a row block
  // are in flight together (and the next block's loads overlap this block's math).
  float alpha = p.alpha;
  if constexpr (FMT == F_E4M3) {
    const int gs = p.sinv_per_group ? grp : 0;           // grouped: one scale per group on both sides
    alpha = (p.a_sinv[gs] * p.b_sinv[gs]) * p.alpha;
  }
  const int64_t c_rows = SCHED == S_GROUP_M ? p.T : p.M;
  const int64_t rows_left = c_rows - m0;
  // Group q (0..3) of 4 consecutive output columns that a lane holds in 32x32 block (i, j):
  // its row and first column within the block, and its 4 values times alpha.
  auto acc_row = [&](int q) { return kM16 ? 16 * (q >> 1) + (lane & 15) : lrow; };
  auto acc_col = [&](int q) { return kM16 ? 16 * (q & 1) + 4 * (lane >> 4) : 8 * q + 4 * lhalf; };
  auto acc_get = [&](int i, int j, int q, float a) {
    if constexpr (kM16)
      return make_float4(a * acc4[i][j][q][0], a * acc4[i][j][q][1], a * acc4[i][j][q][2], a * acc4[i][j][q][3]);
    else
      return make_float4(a * acc[i][j][4 * q + 0], a * acc[i][j][4 * q + 1], a * acc[i][j][4 * q + 2],
                         a * acc[i][j][4 * q + 3]);
  };
  // Row-partitioned MXFP8 activation epilogues with qt_out also write their bf16 output
  // token-blocked (the grouped wgrad operand): after a pass's items, each bf16 result sits in
  // the staged tile over the fp32 values it came from (every thread overwrites only what it
  // read), and threads then quantize it down the columns, 32 rows per block. A tile starts on
  // its group's first row or a multiple of BM rows later, so its rows are positions
  // colt_pos0 + row of the group's 128-aligned range; a pass at or past colt_rows (the group's
  // rows in the tile rounded up to 128) belongs to the next group and is not written, the rest
  // of the range is padding quantized from zeros.
  constexpr bool kColT = FMT == F_MX && SCHED == S_GROUP_M && EPI != E_STORE;
  const bool colq = kColT && p.qt_out != nullptr;
  int64_t colt_pos0 = 0;
  int colt_rows = 0;
  if (colq) {
    colt_pos0 = p.mx_layout[p.G + 1 + grp] + (m0 - grp_lo);
    const int64_t rem = row_end - m0;
    colt_rows = rem >= BM ? BM : (int)((rem + 127) & ~(int64_t)127);
  }
  // The staged epilogues run two passes of 128 rows (rows 0-63 of a pass in LDS half0, 64-127
  // in half1). These kernels take 128 consecutive rows per pass (wave row `pass` stages all its
  // fragments), so each column's 128 codes of a pass fill one whole 128-byte line within the
  // pass: measured, lines completed a pass apart cost far more than the codes themselves. The
  // others take half of each wave row's rows per pass. Row of the tile of pass row rp:
  constexpr bool kContig = kColT;
  auto pass_row = [&](int pass, int rp) {
    return kContig ? pass * WM + rp : (rp >> 6) * WM + pass * (WM / 2) + (rp & 63);
  };
  // A pass's run of codes for output column col is written: inside the tile's part of the
  // group's range and of the ld_t columns.
  auto colt_ok = [&](int64_t col, int pass) {
    const int64_t pos = colt_pos0 + pass * WM;
    return col < n_end && pass * WM < colt_rows && pos >= 0 && pos + WM <= p.ld_t;
  };

  if constexpr (EPI == E_STORE || EPI == E_SRELU) {
    // Two passes over half of each wave's rows: alpha*acc (fp32) goes to LDS in row-major
    // order (16-byte granule g of row r at g ^ (r & 15), conflict-free from the fragment
    // layout), then every thread takes 8 consecutive columns of a row: one 16-byte residual
    // load and one 16-byte store, so each wave moves whole 128-byte lines.
    // E_SRELU (scaled squared ReLU, elementwise): y = p * max(v, 0)^2 goes to c and the
    // pre-activation v (bf16) to aux, at the same offsets (ld_aux == ldc).
    constexpr bool kSR = EPI == E_SRELU;
    static_assert(BM == 2 * WM && NST * STAGE == 2 * 64 * BN * 4, "epilogue staging assumes 2 wave rows");
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(cptr ? cptr + m0 * p.ldc : cptr, cptr ? rows_left * p.ldc * 2 : 0);
    // E_SRELU with q_out: y also as MXFP8 rowwise (ld_q == ldc, so byte offsets are offs / 2; four
    // adjacent lanes hold a 32-column block); E4M3: the group's amax of y (as in E_SWIGLU).
    const bool mxq = kSR && p.q_out != nullptr;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(mxq ? p.q_out + m0 * p.ld_q : p.q_out, mxq ? rows_left * p.ld_q : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(mxq ? p.s_out + m0 * (p.ld_q / 32) : p.s_out,
                                                mxq ? rows_left * (p.ld_q / 32) : 0);
    constexpr bool kAmax = kSR && FMT == F_E4M3;
    float amax_acc = 0.0f;
    if (kAmax && threadIdx.x == 0) amax_slot = 0;
    constexpr int kChunks = BN / 8;                        // 8-column chunks per row
    constexpr int kIters = 128 * kChunks / (NWAVES * 64);  // chunks per thread per pass
    float* stage = reinterpret_cast<float*>(wm ? half1 : half0);
    // Output offset of a thread's item it of a pass (kOOB out of range); held across the
    // epilogue except with the token-blocked output, whose kernels keep every accumulator
    // live longer and recompute it instead.
    auto out_off = [&](int pass, int it) {
      const int id = it * NWAVES * 64 + threadIdx.x;
      const int brow = pass_row(pass, id / kChunks);
      const int64_t n = n0 + (id % kChunks) * 8;
      return (m0 + brow < row_end && n < n_end) ? (int)(((int64_t)brow * p.ldc + n) * 2) : (int)kOOB;
    };
    // The residual of both passes is requested first: its HBM latency overlaps the staging.
    v4i res[2][kIters];
    int offs[2][kIters];
#pragma unroll
    for (int pass = 0; pass < 2; ++pass)
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int rp = id / kChunks;                       // row of the pass (0..127)
        const int brow = pass_row(pass, rp);
        if constexpr (!kContig) offs[pass][it] = out_off(pass, it);
        if (!kSR && p.accumulate) res[pass][it] = __builtin_amdgcn_raw_buffer_load_b128(rc, offs[pass][it], 0, 0);
        if constexpr (kSR)                                 // the row's scale p (res[.][.][0] carries it)
          res[pass][it][0] = __builtin_amdgcn_raw_buffer_load_b32(
              make_rsrc(p.probs + m0, rows_left * 4), m0 + brow < row_end ? brow * 4 : (int)kOOB, 0, 0);
      }
    __syncthreads();                                       // every wave is done with the LDS stages
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int il = 0; il < (kContig ? WMF : WMF / 2); ++il) {
        const int i = kContig ? il : pass * (WMF / 2) + il;
        float* const st = kContig ? reinterpret_cast<float*>(il >= WMF / 2 ? half1 : half0) : stage;
        const int rb = (kContig ? il % (WMF / 2) : il) * 32;
        if (!kContig || wm == pass) {
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = rb + acc_row(q);                 // row within its LDS half
            const int g = (wn * WN + j * 32 + acc_col(q)) >> 2;
            const float4 v = acc_get(i, j, q, alpha);
            *reinterpret_cast<float4*>(st + r * BN + ((g ^ (r & 15)) << 2)) = v;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int rp = id / kChunks, c = id % kChunks;
        const float* row = reinterpret_cast<const float*>(rp >= 64 ? half1 : half0) + (rp & 63) * BN;
        const int sw = (rp & 63) & 15;
        const int off = kContig ? out_off(pass, it) : offs[pass][it];
        const float4 lo = *reinterpret_cast<const float4*>(row + (((2 * c) ^ sw) << 2));
        const float4 hi = *reinterpret_cast<const float4*>(row + (((2 * c + 1) ^ sw) << 2));
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if constexpr (kSR) {
          const float pm = __builtin_bit_cast(float, res[pass][it][0]);
          const v4i vh = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3]), (int)pack_bf16x2(v[4], v[5]),
                          (int)pack_bf16x2(v[6], v[7])};
          __builtin_amdgcn_raw_buffer_store_b128(       // no pre-activation buffer: a zero-size resource
              vh, make_rsrc(p.aux ? p.aux + m0 * p.ld_aux : p.aux, p.aux ? rows_left * p.ld_aux * 2 : 0),
              off, 0, 0);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float rl = fmaxf(v[e], 0.0f);
            v[e] = pm * rl * rl;
          }
        } else if (p.accumulate) {
          const v4i r4 = res[pass][it];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] = bf16_lo((uint32_t)r4[e]) + v[2 * e];
            v[2 * e + 1] = bf16_hi((uint32_t)r4[e]) + v[2 * e + 1];
          }
        }
        const v4i w = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3]), (int)pack_bf16x2(v[4], v[5]),
                       (int)pack_bf16x2(v[6], v[7])};
        __builtin_amdgcn_raw_buffer_store_b128(w, rc, off, 0, 0);
        if constexpr (kSR) {
          if constexpr (kAmax) {
#pragma unroll
            for (int e = 0; e < 8; ++e) amax_acc = fmaxf(amax_acc, fabsf(v[e]));
          }
          if (mxq) {
            const int id = it * NWAVES * 64 + threadIdx.x;
            const int c = id % kChunks;
            int e8;
            const v2i qv = mx_quant_lane8(w, e8);          // every lane takes part
            const int o = off;
            __builtin_amdgcn_raw_buffer_store_b64(qv, rq, o == (int)kOOB ? (int)kOOB : o >> 1, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((char)e8, rs, (o == (int)kOOB || (c & 3)) ? (int)kOOB : o >> 6, 0, 0);
          }
          if constexpr (kColT) {
            if (colq)                                      // y over its first fp32 granule (zero outside)
              *reinterpret_cast<float4*>(const_cast<float*>(row) + (((2 * c) ^ sw) << 2)) =
                  __builtin_bit_cast(float4, off != (int)kOOB ? w : v4i{0, 0, 0, 0});
          }
        }
      }
      if constexpr (kSR && kColT) {
        if (colq) {
          __syncthreads();                                 // the pass's y is in the staged tile
          // columns nl, nl + 1; lanes 0-31 take blocks 0-1 of the pass, lanes 32-63 blocks 2-3
          const int nl = 64 * wave + 2 * (lane & 31);
          mx_colT_run<BN, 2>(half0, half1, 2 * (nl >> 3), (nl & 7) >> 1, 2 * (lane >> 5), p.qt_out, p.st_out, p.ld_t,
                             n0 + nl, colt_pos0 + pass * WM, colt_ok(n0 + nl, pass));
        }
      }
      if (pass == 0) __syncthreads();                      // stage reused by the second pass
    }
    if constexpr (kAmax) {
      if (p.amax_out) {
        amax_to_slot(&amax_slot, amax_acc);
        slot_to_group(&amax_slot, p.amax_out, grp);
      }
    }
  } else if constexpr (glu_fwd(EPI)) {
    // Staged like E_STORE: alpha*acc (each wave column holds WN/2 gate columns a, then the
    // matching WN/2 up columns b) goes to LDS, then each thread takes 8 consecutive output
    // columns of one row: y = p * silu(a) * b, and 16-byte stores of bf16 y and of the two
    // halves of the saved pre-activation. The granule XOR includes the wave column, so the
    // 16 chunks of a row read 16 distinct bank groups.
    // With q_out, y is also emitted as MXFP8 rowwise (E4M3 bytes plus one E8M0 exponent per
    // 32 columns): the MX quantization of bf16(y), exactly as the standalone quantizer would
    // produce it from the bf16 output (four adjacent lanes hold one 32-column block).
    static_assert(BM == 2 * WM && NST * STAGE == 2 * 64 * BN * 4, "epilogue staging assumes 2 wave rows");
    static_assert(WNF % 2 == 0 && BN / 16 == 16, "gate and up fragments per wave column; 16 chunks per row");
    const int64_t ybytes = cptr ? rows_left * p.ldc * 2 : 0;
    const __amdgpu_buffer_rsrc_t ry = make_rsrc(cptr ? cptr + m0 * p.ldc : cptr, ybytes);
    const int64_t hbytes = p.aux ? rows_left * p.ld_aux * 2 : 0;
    const __amdgpu_buffer_rsrc_t rha = make_rsrc(p.aux ? p.aux + m0 * p.ld_aux : p.aux, hbytes);
    const __amdgpu_buffer_rsrc_t rhb = make_rsrc(p.aux ? p.aux + m0 * p.ld_aux + p.F : p.aux, hbytes - p.F * 2);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.probs + m0, rows_left * 4);
    const bool mxq = p.q_out != nullptr;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(mxq ? p.q_out + m0 * p.ld_q : p.q_out, mxq ? rows_left * p.ld_q : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(mxq ? p.s_out + m0 * (p.ld_q / 32) : p.s_out,
                                                mxq ? rows_left * (p.ld_q / 32) : 0);
    constexpr int kChunks = BN / 16;                       // 8-column output chunks per row
    constexpr int kCpw = WN / 16, kGpw = WN / 4;           // chunks, granules per wave column
    constexpr int kIters = 128 * kChunks / (NWAVES * 64);
    auto wsw = [](int w) { return (w & 1) | ((w & 2) << 2); };
    float* stage = reinterpret_cast<float*>(wm ? half1 : half0);
    constexpr bool kAmax = FMT == F_E4M3;                  // per-group amax of y (FP8 current scaling)
    float amax_acc = 0.0f;                                 // max |y| (masked lanes hold 0)
    if (kAmax && threadIdx.x == 0) amax_slot = 0;
    __syncthreads();                                       // every wave is done with the LDS stages
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int il = 0; il < (kContig ? WMF : WMF / 2); ++il) {
        const int i = kContig ? il : pass * (WMF / 2) + il;
        float* const st = kContig ? reinterpret_cast<float*>(il >= WMF / 2 ? half1 : half0) : stage;
        const int rb = (kContig ? il % (WMF / 2) : il) * 32;
        if (!kContig || wm == pass) {
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = rb + acc_row(q);
            const int g = (wn * WN + j * 32 + acc_col(q)) >> 2;
            const float4 v = acc_get(i, j, q, alpha);
            *reinterpret_cast<float4*>(st + r * BN + ((g ^ (r & 15) ^ wsw(wn)) << 2)) = v;
          }
        }
      }
      __syncthreads();
      float pr[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int brow = pass_row(pass, id / kChunks);
        pr[it] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rp, m0 + brow < row_end ? brow * 4 : (int)kOOB, 0, 0));
      }
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int rp_ = id / kChunks, c = id % kChunks;
        // output offsets (out-of-range: kOOB), computed here rather than held across the loop
        const int brow = pass_row(pass, rp_);
        const int64_t n = n0 + c * 8;
        const bool ok = m0 + brow < row_end && n < n_end;
        const int oy = ok ? (int)(((int64_t)brow * p.ldc + n) * 2) : (int)kOOB;
        const int oh = ok ? (int)(((int64_t)brow * p.ld_aux + n) * 2) : (int)kOOB;
        const int oq = ok ? (int)((int64_t)brow * p.ld_q + n) : (int)kOOB;
        const int os = (ok && (c & 3) == 0) ? (int)((int64_t)brow * (p.ld_q / 32) + (n >> 5)) : (int)kOOB;
        const int rr = rp_ & 63, wc = c / kCpw, cc = c % kCpw;
        const float* row = reinterpret_cast<const float*>(rp_ >= 64 ? half1 : half0) + rr * BN;
        const int x = (rr & 15) ^ wsw(wc);
        const int ga = wc * kGpw + 2 * cc, gb = ga + kGpw / 2;   // gate and up granules of this chunk
        const float4 a0 = *reinterpret_cast<const float4*>(row + ((ga ^ x) << 2));
        const float4 a1 = *reinterpret_cast<const float4*>(row + (((ga + 1) ^ x) << 2));
        const float4 b0 = *reinterpret_cast<const float4*>(row + ((gb ^ x) << 2));
        const float4 b1 = *reinterpret_cast<const float4*>(row + (((gb + 1) ^ x) << 2));
        const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const float pm = pr[it];
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if constexpr (EPI == E_CSWIGLU) {
            // clamped: gate min(a, limit) through u * sigmoid(act_alpha * u), up clamp(b) + 1
            const float ac = fminf(a[e], p.act_limit);
            const float bc = __builtin_amdgcn_fmed3f(b[e], -p.act_limit, p.act_limit) + 1.0f;
            y[e] = pm * (ac * fast_sigmoid(p.act_alpha * ac)) * bc;
          } else {
            y[e] = pm * (a[e] * fast_sigmoid(a[e])) * b[e];
          }
        }
        const v4i va = {(int)pack_bf16x2(a[0], a[1]), (int)pack_bf16x2(a[2], a[3]), (int)pack_bf16x2(a[4], a[5]),
                        (int)pack_bf16x2(a[6], a[7])};
        const v4i vb = {(int)pack_bf16x2(b[0], b[1]), (int)pack_bf16x2(b[2], b[3]), (int)pack_bf16x2(b[4], b[5]),
                        (int)pack_bf16x2(b[6], b[7])};
        const v4i vy = {(int)pack_bf16x2(y[0], y[1]), (int)pack_bf16x2(y[2], y[3]), (int)pack_bf16x2(y[4], y[5]),
                        (int)pack_bf16x2(y[6], y[7])};
        __builtin_amdgcn_raw_buffer_store_b128(va, rha, oh, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vb, rhb, oh, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(vy, ry, oy, 0, 0);
        if constexpr (kAmax) {
#pragma unroll
          for (int e = 0; e < 8; ++e) amax_acc = fmaxf(amax_acc, fabsf(y[e]));
        }
        if (mxq) {
          int e8;
          const v2i qv = mx_quant_lane8(vy, e8);
          __builtin_amdgcn_raw_buffer_store_b64(qv, rq, oq, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8((char)e8, rs, os, 0, 0);
        }
        if constexpr (kColT) {
          if (colq)                                        // y over the gate's first granule (zero outside)
            *reinterpret_cast<float4*>(const_cast<float*>(row) + ((ga ^ x) << 2)) =
                __builtin_bit_cast(float4, ok ? vy : v4i{0, 0, 0, 0});
        }
      }
      if constexpr (kColT) {
        if (colq) {
          static_assert(WGN == 2 && kCpw == 8, "two wave columns of 8 output chunks");
          __syncthreads();                                 // the pass's y is in the staged tile
          // Wave w: block w of the pass; lane l: output columns 2l, 2l + 1. Per row the 64 lanes
          // read 16 distinct granules (the wave columns' XORs differ in bit 0).
          const int yc = 2 * lane, wc = yc / (8 * kCpw);
          const int gran = (wc * kGpw + 2 * ((yc >> 3) % kCpw)) ^ wsw(wc);
          mx_colT_run<BN, 1>(half0, half1, gran, (yc & 7) >> 1, wave, p.qt_out, p.st_out, p.ld_t, n0 + yc,
                             colt_pos0 + pass * WM, colt_ok(n0 + yc, pass));
        }
      }
      if (pass == 0) __syncthreads();                      // stage reused by the second pass
    }
    if constexpr (kAmax) {
      if (p.amax_out) {
        amax_to_slot(&amax_slot, amax_acc);
        slot_to_group(&amax_slot, p.amax_out, grp);
      }
    }
  } else {  // E_DSWIGLU, E_DSRELU, E_DCSWIGLU
    // Staged like E_STORE: g = alpha*acc for half of each wave's rows goes to LDS, then each
    // thread takes 8 consecutive columns of one row: 16-byte loads of a and b (the two halves
    // of the saved pre-activation), 16-byte stores of da and db. A row's BN/8 chunks are 32
    // consecutive lanes, which reduce the row's dprobs partial in a fixed order; one partial
    // per row and column tile goes to the workspace.
    static_assert(BM == 2 * WM && NST * STAGE == 2 * 64 * BN * 4, "epilogue staging assumes 2 wave rows");
    static_assert(BN / 8 == 32, "a row's chunks fill half a wave");
    // E_DSRELU (scaled squared ReLU): one pre-activation h [T, F]; dh = g * p * 2 max(h, 0),
    // dprobs partial sum of g * max(h, 0)^2.
    constexpr bool kSR = EPI == E_DSRELU;
    // E_DCSWIGLU (clamped SwiGLU): the gate's gradient passes where a <= limit, the up half's
    // where |b| <= limit (a clamp passes it inside its closed interval), from the clamped values.
    constexpr bool kCl = EPI == E_DCSWIGLU;
    const int64_t hbytes = rows_left * p.ld_aux * 2;
    const int64_t dbytes = p.aux_out ? rows_left * p.ld_aux_out * 2 : 0;
    // One resource per tensor; the b half sits F columns further (an out-of-range offset
    // stays out of range when that is added).
    const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.aux + m0 * p.ld_aux, hbytes);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.aux_out ? p.aux_out + m0 * p.ld_aux_out : p.aux_out, dbytes);
    const int fb = (int)(p.F * 2);                         // byte distance of the b half (bf16)
    // With q_out, dact is also emitted as MXFP8 rowwise (blocks of 32 along 2F, which never
    // straddle the da / db halves as F % 32 == 0), the bytes the standalone quantizer writes
    // for the bf16 dact. Its row stride ld_q equals ld_aux_out, so byte offsets are od / 2.
    const bool mxq = p.q_out != nullptr;
    constexpr bool kAmax = FMT == F_E4M3;                  // per-group amax of dh (FP8 current scaling)
    const bool want_amax = kAmax && p.amax_out != nullptr;
    if (want_amax && threadIdx.x == 0) amax_slot = 0;       // before the epilogue's first barrier
    const int64_t qbytes = mxq ? rows_left * p.ld_q : 0, sbytes = mxq ? rows_left * (p.ld_q / 32) : 0;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(mxq ? p.q_out + m0 * p.ld_q : p.q_out, qbytes);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(mxq ? p.s_out + m0 * (p.ld_q / 32) : p.s_out, sbytes);
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(p.probs + m0, rows_left * 4);
    const __amdgpu_buffer_rsrc_t rpart = make_rsrc(p.dp_part + (int64_t)nt * p.T + m0, rows_left * 4);
    constexpr int kChunks = BN / 8;
    constexpr int kIters = 128 * kChunks / (NWAVES * 64);
    float* stage = reinterpret_cast<float*>(wm ? half1 : half0);
    __syncthreads();                                       // every wave is done with the LDS stages
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int il = 0; il < (kContig ? WMF : WMF / 2); ++il) {
        const int i = kContig ? il : pass * (WMF / 2) + il;
        float* const st = kContig ? reinterpret_cast<float*>(il >= WMF / 2 ? half1 : half0) : stage;
        const int rb = (kContig ? il % (WMF / 2) : il) * 32;
        if (!kContig || wm == pass) {
#pragma unroll
        for (int j = 0; j < WNF; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int r = rb + acc_row(q);
            const int g = (wn * WN + j * 32 + acc_col(q)) >> 2;
            const float4 v = acc_get(i, j, q, alpha);
            *reinterpret_cast<float4*>(st + r * BN + ((g ^ (r & 15)) << 2)) = v;
          }
        }
      }
      __syncthreads();
      // Chunks go in batches of SGE_DSWIGLU_BATCH (all loads of a batch in flight together),
      // which bounds the live registers when one thread owns 8 or 16 chunks; 4 measured 4%
      // faster than 8 on the FP8 grouped dgrad and the same elsewhere.
      constexpr int kBatch = kIters < SGE_DSWIGLU_BATCH ? kIters : SGE_DSWIGLU_BATCH;
      static_assert(kIters % kBatch == 0, "whole batches");
#pragma unroll
      for (int it0 = 0; it0 < kIters; it0 += kBatch) {
      v4i ha[kBatch], hb[kBatch];
      float pr[kBatch];
      int oh[kBatch], od[kBatch], orow[kBatch];
#pragma unroll
      for (int ib = 0; ib < kBatch; ++ib) {
        const int it = it0 + ib;
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int rp_ = id / kChunks, c = id % kChunks;
        const int brow = pass_row(pass, rp_);
        const int64_t n = n0 + c * 8;
        const bool rok = m0 + brow < row_end;
        const bool ok = rok && n < n_end;
        oh[ib] = ok ? (int)(((int64_t)brow * p.ld_aux + n) * 2) : (int)kOOB;
        od[ib] = ok ? (int)(((int64_t)brow * p.ld_aux_out + n) * 2) : (int)kOOB;
        orow[ib] = rok ? brow * 4 : (int)kOOB;
        ha[ib] = __builtin_amdgcn_raw_buffer_load_b128(rh, oh[ib], 0, 0);
        if constexpr (!kSR) hb[ib] = __builtin_amdgcn_raw_buffer_load_b128(rh, oh[ib] + fb, 0, 0);
        pr[ib] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rp, orow[ib], 0, 0));
      }
#pragma unroll
      for (int ib = 0; ib < kBatch; ++ib) {
        const int it = it0 + ib;
        const int id = it * NWAVES * 64 + threadIdx.x;
        const int rp_ = id / kChunks, c = id % kChunks;
        const float* row = reinterpret_cast<const float*>(rp_ >= 64 ? half1 : half0) + (rp_ & 63) * BN;
        const int sw = (rp_ & 63) & 15;
        const float4 lo = *reinterpret_cast<const float4*>(row + (((2 * c) ^ sw) << 2));
        const float4 hi = *reinterpret_cast<const float4*>(row + (((2 * c + 1) ^ sw) << 2));
        const float g[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const float pm = pr[ib];
        float da[8], db[8], part = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t wa = (uint32_t)ha[ib][e >> 1];
          const float a = (e & 1) ? bf16_hi(wa) : bf16_lo(wa);
          if constexpr (kSR) {
            const float rl = fmaxf(a, 0.0f);
            da[e] = g[e] * pm * 2.0f * rl;
            db[e] = 0.0f;
            part += g[e] * rl * rl;
          } else if constexpr (kCl) {
            const uint32_t wb = (uint32_t)hb[ib][e >> 1];
            const float b = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
            const float lim = p.act_limit, al = p.act_alpha;
            const float ac = fminf(a, lim);
            const float bc = __builtin_amdgcn_fmed3f(b, -lim, lim) + 1.0f;
            const float sg = fast_sigmoid(al * ac);
            const float q = ac * sg;
            const float dq = sg * (1.0f + al * ac * (1.0f - sg));
            da[e] = a <= lim ? g[e] * pm * bc * dq : 0.0f;
            db[e] = fabsf(b) <= lim ? g[e] * pm * q : 0.0f;
            part += g[e] * q * bc;
          } else {
            const uint32_t wb = (uint32_t)hb[ib][e >> 1];
            const float b = (e & 1) ? bf16_hi(wb) : bf16_lo(wb);
            const float sg = fast_sigmoid(a);
            const float silu = a * sg;
            const float dsilu = sg * (1.0f + a * (1.0f - sg));
            da[e] = g[e] * pm * b * dsilu;
            db[e] = g[e] * pm * silu;
            part += g[e] * silu * b;
          }
        }
        const v4i va = {(int)pack_bf16x2(da[0], da[1]), (int)pack_bf16x2(da[2], da[3]),
                        (int)pack_bf16x2(da[4], da[5]), (int)pack_bf16x2(da[6], da[7])};
        const v4i vb = {(int)pack_bf16x2(db[0], db[1]), (int)pack_bf16x2(db[2], db[3]),
                        (int)pack_bf16x2(db[4], db[5]), (int)pack_bf16x2(db[6], db[7])};
        __builtin_amdgcn_raw_buffer_store_b128(va, rd, od[ib], 0, 0);
        if constexpr (!kSR) __builtin_amdgcn_raw_buffer_store_b128(vb, rd, od[ib] + fb, 0, 0);
        if constexpr (kAmax) {
          if (want_amax) {                                 // per item: no register lives across items
            float mi = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) mi = fmaxf(mi, fmaxf(fabsf(da[e]), fabsf(db[e])));   // db = 0 for SReLU
            amax_to_slot(&amax_slot, mi);
          }
        }
        if (mxq) {
          int ea;
          const v2i qa = mx_quant_lane8(va, ea);
          const int oq = od[ib] == (int)kOOB ? (int)kOOB : od[ib] >> 1;
          const int os = (od[ib] == (int)kOOB || (c & 3)) ? (int)kOOB : od[ib] >> 6;
          __builtin_amdgcn_raw_buffer_store_b64(qa, rq, oq, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8((char)ea, rs, os, 0, 0);
          if constexpr (!kSR) {
            int eb;
            const v2i qb = mx_quant_lane8(vb, eb);
            __builtin_amdgcn_raw_buffer_store_b64(qb, rq, oq + fb / 2, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b8((char)eb, rs, os + fb / 64, 0, 0);
          }
        }
        if constexpr (kColT) {
          if (colq) {                                      // da, db over their fp32 granules (zero outside)
            const bool okw = od[ib] != (int)kOOB;
            float* wrow = const_cast<float*>(row);
            *reinterpret_cast<float4*>(wrow + (((2 * c) ^ sw) << 2)) =
                __builtin_bit_cast(float4, okw ? va : v4i{0, 0, 0, 0});
            if constexpr (!kSR)
              *reinterpret_cast<float4*>(wrow + (((2 * c + 1) ^ sw) << 2)) =
                  __builtin_bit_cast(float4, okw ? vb : v4i{0, 0, 0, 0});
          }
        }
        // the row's 32 chunks are lanes c = 0..31 of one half-wave: fixed-order tree sum
#pragma unroll
        for (int d = 1; d < 32; d <<= 1) part += __shfl_xor(part, d, 64);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, part), rpart, c == 0 ? orow[ib] : (int)kOOB,
                                              0, 0);
      }
      }
      if constexpr (kColT) {
        if (colq) {
          __syncthreads();                                 // the pass's da / db are in the staged tile
          // Columns nl, nl + 1 of da (lanes 0-31) and of db (32-63, gated activations), all four
          // blocks of the pass; per row a wave reads 16 distinct granules. SReLU (da only): lanes
          // 32-63 take blocks 2-3 instead.
          const int nl = 64 * wave + 2 * (lane & 31);
          const int64_t pos = colt_pos0 + pass * WM;
          const bool ok = colt_ok(n0 + nl, pass);
          if constexpr (kSR) {
            mx_colT_run<BN, 2>(half0, half1, 2 * (nl >> 3), (nl & 7) >> 1, 2 * (lane >> 5), p.qt_out, p.st_out,
                               p.ld_t, n0 + nl, pos, ok);
          } else {
            const int side = lane >> 5;
            mx_colT_run<BN, 4>(half0, half1, 2 * (nl >> 3) + side, (nl & 7) >> 1, 0, p.qt_out, p.st_out, p.ld_t,
                               n0 + nl + (side ? p.F : 0), pos, ok);
          }
        }
      }
      if (pass == 0) __syncthreads();                      // stage reused by the second pass
    }
    if constexpr (kAmax) {
      if (want_amax) slot_to_group(&amax_slot, p.amax_out, grp);
    }
  }
}

template <int FMT, bool AK, bool BK, int EPI, int SCHED, int WGM, int WGN, int WMF, int WNF>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WGM * WGN, 64 * WGM * WGN),
                          amdgpu_waves_per_eu(WGM * WGN / 4, WGM * WGN / 4)))
void gemm_kernel(const GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[131072];
  __shared__ __attribute__((aligned(16))) uint8_t sc[tile_sc_bytes(FMT, SCHED, EPI)];
  __shared__ uint32_t amax_slot;
  gemm_tile<FMT, AK, BK, EPI, SCHED, WGM, WGN, WMF, WNF>(p, blockIdx.x, lds, sc, &amax_slot);
}

// ------------------------------------------------------------------ launchers
template <int FMT, bool AK, bool BK, int EPI, int SCHED, int WGM, int WGN, int WMF, int WNF>
static hipError_t launch_cfg(GemmParams p, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_kernel<FMT, AK, BK, EPI, SCHED, WGM, WGN, WMF, WNF>), dim3(grid), dim3(64 * WGM * WGN), 0,
                     s, p);
  return hipGetLastError();
}

// A GEMM's tile kind: its tile shape, the tile body, and the launch size.
template <int FMT, bool AK, bool BK, int EPI, int SCHED>
struct Kind {
  using TS = TileShape<FMT, SCHED, EPI>;
  static constexpr int WGM = TS::WGM, WGN = TS::WGN, WMF = TS::WMF, WNF = TS::WNF;
  static constexpr int BM = WGM * 32 * WMF, BN = WGN * 32 * WNF;
  static constexpr int kThreads = 64 * WGM * WGN;
  static constexpr int kScBytes = tile_sc_bytes(FMT, SCHED, EPI);
  __device__ __forceinline__ static void run(const GemmParams& p, int blk, uint8_t* lds, uint8_t* sc,
                                             uint32_t* slot) {
    gemm_tile<FMT, AK, BK, EPI, SCHED, WGM, WGN, WMF, WNF>(p, blk, lds, sc, slot);
  }
  // Fills the tile counts of p; returns the number of tiles to launch (an upper bound for the
  // row-partitioned grouped schedule, whose extra tiles return at once).
  static int prepare(GemmParams& p) {
    if constexpr (SCHED == S_DENSE) {
      p.mt_count = (int)((p.M + BM - 1) / BM);
      p.nt_count = (int)((p.N + BN - 1) / BN);
      return p.mt_count * p.nt_count;
    } else if constexpr (SCHED == S_GROUP_M) {
      const int64_t ncols = glu_fwd(EPI) ? p.F : p.N;
      const int64_t ntile = glu_fwd(EPI) ? BN / 2 : BN;
      p.nt_count = (int)((ncols + ntile - 1) / ntile);
      const int64_t mtiles = (p.T + BM - 1) / BM + p.G;   // upper bound over any split
      return (int)(mtiles * p.nt_count);
    } else {
      p.mt_count = (int)((p.M + BM - 1) / BM);
      p.nt_count = (int)((p.N + BN - 1) / BN);
      return p.mt_count * p.nt_count * p.G;
    }
  }
};

template <int FMT, bool AK, bool BK, int EPI, int SCHED>
static hipError_t launch_tile(GemmParams p, hipStream_t s) {
  using K = Kind<FMT, AK, BK, EPI, SCHED>;
  const int grid = K::prepare(p);                        // fills p's tile counts first
  return launch_cfg<FMT, AK, BK, EPI, SCHED, K::WGM, K::WGN, K::WMF, K::WNF>(p, grid, s);
}

// Two independent GEMMs in one launch ("Activation + GroupedLinear Fusion for MOE and other MOE
// optimizations", review discussion: the FC1 - ACT - FC2 module fused): a layer's dgrad beside
// its wgrad. Workgroups go out in groups of 8 (one per XCD): the groups of A, then those of B,
// so the end of A overlaps the start of B instead of each launch draining on its own (the
// grouped MLP backward measured 2% faster per step than with the two launches; interleaving the
// groups of A and B in proportion measured 3% slower, the two GEMMs then sharing each XCD's L2).
// Within a GEMM, group j and XCD x give tile number 8 j + x, the numbering its own launch would
// have. The tiles share the workgroup's LDS (both kinds have the same wave count).
template <class KA, class KB>
__global__ __attribute__((amdgpu_flat_work_group_size(KA::kThreads, KA::kThreads),
                          amdgpu_waves_per_eu(KA::kThreads / 256, KA::kThreads / 256)))
void gemm_pair_kernel(const GemmParams pa, const GemmParams pb, int ga) {
  static_assert(KA::kThreads == KB::kThreads, "one workgroup size");
  __shared__ __attribute__((aligned(16))) uint8_t lds[131072];
  __shared__ __attribute__((aligned(16))) uint8_t sc[KA::kScBytes > KB::kScBytes ? KA::kScBytes : KB::kScBytes];
  __shared__ uint32_t slot;
  const int g = blockIdx.x >> 3, x = blockIdx.x & 7;
  if (g < ga) KA::run(pa, g * 8 + x, lds, sc, &slot);
  else KB::run(pb, (g - ga) * 8 + x, lds, sc, &slot);
}

template <class KA, class KB>
static hipError_t launch_pair(GemmParams pa, GemmParams pb, hipStream_t s) {
  const int na = KA::prepare(pa), nb = KB::prepare(pb);
  if (na <= 0 && nb <= 0) return hipSuccess;
  const int ga = (na + 7) / 8, gb = (nb + 7) / 8;
  hipLaunchKernelGGL((gemm_pair_kernel<KA, KB>), dim3(8 * (ga + gb)), dim3(KA::kThreads), 0, s, pa, pb, ga);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmParams& p, int fmt, bool a_kmaj, bool b_kmaj, hipStream_t s) {
  if (fmt == F_BF16) {
    if (a_kmaj && b_kmaj) return launch_tile<F_BF16, true, true, E_STORE, S_DENSE>(p, s);
    if (a_kmaj && !b_kmaj) return launch_tile<F_BF16, true, false, E_STORE, S_DENSE>(p, s);
    if (!a_kmaj && !b_kmaj) return launch_tile<F_BF16, false, false, E_STORE, S_DENSE>(p, s);
    return launch_tile<F_BF16, false, true, E_STORE, S_DENSE>(p, s);
  }
  if (fmt == F_E4M3) return launch_tile<F_E4M3, true, true, E_STORE, S_DENSE>(p, s);
  if (p.mx_aligned) return launch_tile<F_MX, true, true, E_STORE, S_DENSE>(p, s);
  return launch_tile<F_MXU, true, true, E_STORE, S_DENSE>(p, s);
}

hipError_t launch_grouped_fwd(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_SWIGLU) return launch_tile<F_BF16, true, true, E_SWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_SRELU) return launch_tile<F_BF16, true, true, E_SRELU, S_GROUP_M>(p, s);
  if (epilogue == E_CSWIGLU) return launch_tile<F_BF16, true, true, E_CSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_BF16, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_fwd_mx(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_SWIGLU) return launch_tile<F_MX, true, true, E_SWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_SRELU) return launch_tile<F_MX, true, true, E_SRELU, S_GROUP_M>(p, s);
  if (epilogue == E_CSWIGLU) return launch_tile<F_MX, true, true, E_CSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_MX, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_dgrad(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_DSWIGLU) return launch_tile<F_BF16, true, false, E_DSWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_DSRELU) return launch_tile<F_BF16, true, false, E_DSRELU, S_GROUP_M>(p, s);
  if (epilogue == E_DCSWIGLU) return launch_tile<F_BF16, true, false, E_DCSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_BF16, true, false, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_wgrad(const GemmParams& p, hipStream_t s) {
  return launch_tile<F_BF16, false, false, E_STORE, S_GROUP_K>(p, s);
}

hipError_t launch_grouped_dgrad_wgrad(const GemmParams& dg, int epilogue, const GemmParams& wg, hipStream_t s) {
  using W = Kind<F_BF16, false, false, E_STORE, S_GROUP_K>;
  if (epilogue == E_DSWIGLU) return launch_pair<Kind<F_BF16, true, false, E_DSWIGLU, S_GROUP_M>, W>(dg, wg, s);
  if (epilogue == E_DSRELU) return launch_pair<Kind<F_BF16, true, false, E_DSRELU, S_GROUP_M>, W>(dg, wg, s);
  if (epilogue == E_DCSWIGLU) return launch_pair<Kind<F_BF16, true, false, E_DCSWIGLU, S_GROUP_M>, W>(dg, wg, s);
  return launch_pair<Kind<F_BF16, true, false, E_STORE, S_GROUP_M>, W>(dg, wg, s);
}

hipError_t launch_grouped_fwd_fp8(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_SWIGLU) return launch_tile<F_E4M3, true, true, E_SWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_SRELU) return launch_tile<F_E4M3, true, true, E_SRELU, S_GROUP_M>(p, s);
  if (epilogue == E_CSWIGLU) return launch_tile<F_E4M3, true, true, E_CSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_E4M3, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_dgrad_fp8(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_DSWIGLU) return launch_tile<F_E4M3, true, true, E_DSWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_DSRELU) return launch_tile<F_E4M3, true, true, E_DSRELU, S_GROUP_M>(p, s);
  if (epilogue == E_DCSWIGLU) return launch_tile<F_E4M3, true, true, E_DCSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_E4M3, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_wgrad_fp8(const GemmParams& p, hipStream_t s) {
  return launch_tile<F_E4M3, true, true, E_STORE, S_GROUP_K>(p, s);
}

hipError_t launch_grouped_dgrad_mx(const GemmParams& p, int epilogue, hipStream_t s) {
  if (epilogue == E_DSWIGLU) return launch_tile<F_MX, true, true, E_DSWIGLU, S_GROUP_M>(p, s);
  if (epilogue == E_DSRELU) return launch_tile<F_MX, true, true, E_DSRELU, S_GROUP_M>(p, s);
  if (epilogue == E_DCSWIGLU) return launch_tile<F_MX, true, true, E_DCSWIGLU, S_GROUP_M>(p, s);
  return launch_tile<F_MX, true, true, E_STORE, S_GROUP_M>(p, s);
}

hipError_t launch_grouped_wgrad_mx(const GemmParams& p, hipStream_t s) {
  return launch_tile<F_MX, true, true, E_STORE, S_GROUP_K>(p, s);
}

int gemm_tile_n() { return kWavesN * 32 * kFragsN; }
int gemm_dp_parts_per_tile() { return 1; }

}  // namespace sge
