// Device-side building blocks shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// log2(e) and ln(2): the kernels keep scores in the base-2 domain
// (s * scale * log2 e) so that every exponential is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(uint32_t(h) << 16);
}

// Two floats to two bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 f = {a, b};
  bf16x2 h = __builtin_convertvector(f, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float a) {
  return uint16_t(pack_bf16x2(a, 0.f) & 0xffffu);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D = A(32x16) * B(16x32) + C, bf16 in, f32 accumulate.  Lane l holds
// A[l%32][8*(l/32) .. +7], B[8*(l/32) .. +7][l%32] and
// C[8*(i/4) + 4*(l/32) + i%4][l%32] for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Row index of accumulator element i for a lane in half-wave g (32x32 tile).
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Swap bits 2 and 3 of a row index within a 32-row block.  Feeding MFMA row r
// from physical row swap23(r) makes the eight accumulator rows a lane holds
// for i = 8c .. 8c+7 the contiguous physical rows 16c + 8g .. 16c + 8g + 7,
// so a score tile can be used directly as the k-operand of the next product.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~0xc) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value, so that addresses derived from it stay in scalar registers.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// Lane exchange with the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max(x, x of the lane 32 away) and x + (x of the lane 32 away), using the
// VALU half-wave swap: after the swap one register holds the low half-wave's
// values in both halves and the other the high half-wave's, so the
// combination is the same in every lane.
__device__ __forceinline__ float halfwave_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halfwave_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane L supplies the address of 4 consecutive bf16 that form row L/4,
// columns 4*(L%4) .. 4*(L%4)+3 of a 4 x 16 block; lane j receives column j
// of that block (its 4 rows, in row order).
__device__ __forceinline__ u32x2 lds_tr4(const uint16_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uint16_t*)p);
  return __builtin_bit_cast(u32x2, v);
}

// Per-lane offset (in elements) for tr_col8 within a row-major LDS tile of
// the given pitch.
__device__ __forceinline__ int tr_lane_offset(int lane, int pitch) {
  return ((lane >> 2) & 3) * pitch + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
}

// k-operand of a 32x32x16 MFMA contracted over 8 consecutive ROWS of a
// row-major LDS tile: lane l gets rows r0 .. r0+7 (r0 = base + 8*(l/32),
// uniform per 16-lane group) of column c0 + l%32.  `p` = tile + r0*pitch +
// c0 + tr_lane_offset(lane, pitch).
__device__ __forceinline__ u32x4 tr_col8(const uint16_t* p, int pitch) {
  const u32x2 a = lds_tr4(p);
  const u32x2 b = lds_tr4(p + 4 * pitch);
  return u32x4{a[0], a[1], b[0], b[1]};
}

// ---------------------------------------------------------------------------
// Swizzled [ROWS][D] bf16 tiles in LDS, filled by global_load_lds.
//
// Rows are dense (D * 2 bytes); within each aligned group of eight 16-byte
// chunks, logical chunk c of row r is stored at chunk c ^ tile_swz(r) with
// tile_swz(r) = 2 (r & 3) | ((r >> 3) & 1).  LDS has 32 banks of 4 bytes
// (128 bytes per cycle), so:
//  * a b128 row read where lanes 0..7 take rows swap23(0..7) =
//    {0,1,2,3,8,9,10,11} (plus a multiple of 32) at one logical chunk hits 8
//    distinct chunk positions of a 128-byte window;
//  * a transpose read where 16 lanes take 4 consecutive rows (starting at a
//    multiple of 4) x 32 bytes hits 4 distinct 32-byte windows.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_swz(int r) { return (2 * (r & 3)) | ((r >> 3) & 1); }

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x3f70); }

// This wave's share of the transfer of rows r0 .. r0+ROWS-1 of a row-major
// [*, D] bf16 matrix (rows at or beyond rlimit read row rlimit-1 instead)
// into the swizzled tile `dst`.  Each global_load_lds moves 64 chunks of 16
// bytes: lane l of block blk fills physical chunk blk*64 + l.
template <int D, int ROWS, int NWAVES>
__device__ __forceinline__ void dma_tile(const uint16_t* src, uint16_t* dst, int r0, int rlimit,
                                         int wave, int lane) {
  constexpr int CPR = D / 8;
  constexpr int BLOCKS = ROWS * D / 512;
  static_assert(BLOCKS % NWAVES == 0, "tile must split evenly over the waves");
  if (r0 + ROWS <= rlimit) {
    // Full tile: a uniform base plus per-lane offsets that do not depend on
    // the tile (addressing with a scalar base and a 32-bit vector offset).
    const uint16_t* base = src + (int64_t)r0 * D;
#pragma unroll
    for (int j = 0; j < BLOCKS / NWAVES; ++j) {
      const int blk = j * NWAVES + wave;
      const int pos = blk * 64 + lane;
      const int r = pos / CPR;
      const int lc = (pos % CPR) ^ tile_swz(r);
      __builtin_amdgcn_global_load_lds((const void*)(base + (r * D + lc * 8)),
                                       (__attribute__((address_space(3))) void*)(dst + blk * 512),
                                       16, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < BLOCKS / NWAVES; ++j) {
      const int blk = j * NWAVES + wave;
      const int pos = blk * 64 + lane;
      const int r = pos / CPR;
      const int lc = (pos % CPR) ^ tile_swz(r);
      const int row = min(r0 + r, rlimit - 1);
      __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)row * D + lc * 8),
                                       (__attribute__((address_space(3))) void*)(dst + blk * 512),
                                       16, 0, 0);
    }
  }
}

// Element offsets, within a swizzled [*, D] tile, of the b128 row read that
// feeds MFMA A-row n of a 32-row block (physical row swap23(n)) with logical
// chunk 2c + g, for c = 0..3; chunk c >= 4 adds 64 * (c / 4) elements.
template <int D>
__device__ __forceinline__ void row_read_offsets(int n, int g, int* off) {
  const int h = (2 * (n & 3)) | ((n >> 2) & 1);  // tile_swz(swap23(n))
#pragma unroll
  for (int c = 0; c < 4; ++c) off[c] = swap23(n) * D + 8 * ((2 * c + g) ^ h);
}

// Element offsets for tr_col8 on a swizzled [*, D] tile when the 8-row group
// starts at a row base + 8g (base a multiple of 16): logical column block
// db (32 columns) with db even (off[0]) or odd (off[1]); block db adds
// 64 * (db / 2) elements.
template <int D>
__device__ __forceinline__ void tr_read_offsets(int lane, int* off) {
  const int g = lane >> 5;
  const int vr = (lane >> 2) & 3;
  const int h = (2 * vr) | g;
  const int lc = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
#pragma unroll
  for (int p = 0; p < 2; ++p) off[p] = (8 * g + vr) * D + 8 * ((4 * p + lc) ^ h) + 4 * (lane & 1);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace attn
