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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Row index of accumulator element i for a lane in half-wave g (32x32 tile).
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Swap bits 2 and 3 of a row index within a 32-row block.  Feeding MFMA row r
// from physical row swap23(r) makes the eight accumulator rows a lane holds
// for i = 8c .. 8c+7 the contiguous physical rows 16c + 8g .. 16c + 8g + 7,
// so a score tile can be used directly as the k-operand of the next product.
__device__ __forceinline__ int swap23(int r) {
  return (r & ~0xc) | ((r & 4) << 1) | ((r & 8) >> 1);
}

}  // namespace attn
