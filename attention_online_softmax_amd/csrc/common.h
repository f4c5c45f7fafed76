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

// DPP lane permutations within rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowRor8 = 0x128;      // row_ror:8 (lane i of a row reads lane (i + 8) % 16)

// Sum (or max) over each aligned group of N consecutive lanes; every lane of
// the group receives the result.  Steps: lane ^ 1, lane ^ 2 (quad perms),
// mirror within 8 and within 16 (each pairs lanes whose partial results
// cover disjoint halves), then lane ^ 16 (permlane16 swap: with both
// operands x, the two results are x and x of lane ^ 16) and lane ^ 32.
template <int N, bool MAX>
__device__ __forceinline__ float group_reduce(float x) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (N >= 2) x = op(x, dpp_mov<kQuadXor1>(x));
  if constexpr (N >= 4) x = op(x, dpp_mov<kQuadXor2>(x));
  if constexpr (N >= 8) x = op(x, dpp_mov<kRowHalfMirror>(x));
  if constexpr (N >= 16) x = op(x, dpp_mov<kRowMirror>(x));
  if constexpr (N >= 32) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (N >= 64) x = MAX ? halfwave_max(x) : halfwave_sum(x);
  return x;
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

// ---------------------------------------------------------------------------
// Swizzled [ROWS][D] bf16 tiles in LDS, filled by loads to LDS.
//
// Rows are dense (D * 2 bytes).  Logical 16-byte chunk k of row r is stored
// at chunk k ^ tile_swz<D>(r); the XOR stays inside aligned groups of 16
// chunks (8 for D = 64).  LDS has 64 banks of 4 bytes (256 bytes per cycle);
// a b128 read is served 16 lanes per cycle and a b64 transpose read 32 lanes
// per cycle.  The swizzle makes both access patterns of the kernels free of
// bank conflicts:
//  * b128 row reads: 16 lanes take the 16 rows of an aligned 16-row group at
//    one logical chunk; tile_swz is a bijection of r & 15 (of bits 1..3 for
//    D = 64, where bit 0 picks the half of the 256-byte bank window);
//  * transpose reads: 32 lanes take 4 consecutive rows (from a multiple of 4)
//    x 64 bytes; bits 3..2 of tile_swz (bit 2 with the row parity for D = 64)
//    place those rows in the 4 distinct 64-byte quarters of the bank window.
// Rows r and r + 4 (r & 4 == 0) differ only in the top bit of the swizzle, so
// the second half of an 8-row transpose read reuses the offset of another
// 32-column block (tr_col8).
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D >= 128)
    return ((((r >> 2) ^ (r >> 1)) & 1) << 3) | ((r & 1) << 2) | (((r >> 3) & 1) << 1) |
           ((r >> 1) & 1);
  else
    return ((((r >> 1) ^ (r >> 2)) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 1) & 1);
}

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x3f70); }

// Compensated (Kahan) running sum of the softmax normaliser; its value is
// s - c.  Tile sums added to a running sum that dwarfs them lose their low
// bits, and when they repeat (many keys with equal scores after a dominant
// one) the loss keeps one sign and grows with the key count; c carries it.
struct KahanSum {
  float s, c;
  __device__ __forceinline__ void scale(float a) {
    s *= a;
    c *= a;
  }
  __device__ __forceinline__ void add(float x) {
    const float y = x - c;
    const float t = s + y;
    c = (t - s) - y;
    s = t;
  }
  __device__ __forceinline__ float value() const { return s - c; }
};

// Workgroup barrier for LDS tiles filled by loads to LDS, without the
// release/acquire fences of __syncthreads (which wait for every load in
// flight, including prefetches of later tiles).  Callers wait for their own
// transfers of the tile (wait_vmcnt) before it; every LDS read issued before
// it has been consumed by then.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Cache policy of a load to LDS: kCacheDefault, or kCacheStream (the
// non-temporal hint) for data read once, such as the key/value cache of a
// decode step, which then does not displace lines that are reused.
constexpr int kCacheDefault = 0;
constexpr int kCacheStream = 2;

// This wave's share of the transfer of rows r0 .. r0+ROWS-1 of a row-major
// [*, D] bf16 matrix (rows at or beyond rlimit read row rlimit-1 instead)
// into the swizzled tile `dst`.  Each global_load_lds moves 64 chunks of 16
// bytes: lane l of block blk fills physical chunk blk*64 + l.
template <int D, int ROWS, int NWAVES, int CPOL = kCacheDefault>
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
      const int lc = (pos % CPR) ^ tile_swz<D>(r);
      __builtin_amdgcn_global_load_lds((const void*)(base + (r * D + lc * 8)),
                                       (__attribute__((address_space(3))) void*)(dst + blk * 512),
                                       16, 0, CPOL);
    }
  } else {
#pragma unroll
    for (int j = 0; j < BLOCKS / NWAVES; ++j) {
      const int blk = j * NWAVES + wave;
      const int pos = blk * 64 + lane;
      const int r = pos / CPR;
      const int lc = (pos % CPR) ^ tile_swz<D>(r);
      const int row = min(r0 + r, rlimit - 1);
      __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)row * D + lc * 8),
                                       (__attribute__((address_space(3))) void*)(dst + blk * 512),
                                       16, 0, CPOL);
    }
  }
}

// Raw buffer resource over `bytes` bytes at `base` (stride 0, 32-bit data
// format word), for loads whose address is a scalar base plus a 32-bit
// per-lane offset.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// The transfer of dma_tile through a buffer resource whose range is the
// whole [rows, D] matrix: the per-lane byte offsets are computed once and a
// tile costs one scalar offset.  Rows at or beyond `rows` fall outside the
// range; the hardware returns zeros for them, so a ragged last tile arrives
// zero-padded.
template <int D, int ROWS, int NWAVES>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int NJ = ROWS * D / 512 / NWAVES;
  static_assert((ROWS * D / 512) % NWAVES == 0, "tile must split evenly over the waves");
  int voff[NJ];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int pos = (j * NWAVES + wave) * 64 + lane;
      const int r = pos / CPR;
      const int lc = (pos % CPR) ^ tile_swz<D>(r);
      voff[j] = (r * D + lc * 8) * 2;
    }
  }
  // Rows r0 .. r0+ROWS-1 of the [rows, D] bf16 matrix at `src` into `dst`.
  template <int CPOL = kCacheDefault>
  __device__ __forceinline__ void load(const uint16_t* src, int rows, uint16_t* dst, int r0,
                                       int wave) const {
    const rsrc_t rs = make_rsrc(src, (uint32_t)rows * D * 2);
    const int soff = (int)((uint32_t)r0 * D * 2);   // byte offset, may pass 2^31
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      // (a local copy: passing voff[j] straight to the builtin makes the
      // host pass drop the launch stubs of some kernel instantiations)
      const int vo = voff[j];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(dst + (j * NWAVES + wave) * 512), 16, vo,
          soff, 0, CPOL);
    }
  }
};

// Per-lane byte offsets into a swizzled [*, D] tile.  The XOR group is 16
// chunks (128 elements), so D = 256 keeps the offsets of its first 128
// columns in registers and adds 256 bytes for the rest.  Byte offsets are
// added to the tile's address as they are (no shift per read).
template <int D>
constexpr int kRowOffs = D >= 256 ? 8 : D / 16;
template <int D>
constexpr int kTrOffs = D >= 256 ? 4 : D / 32;

// 16-byte LDS read at byte offset `boff` from the tile at `base`.
__device__ __forceinline__ u32x4 lds_row(const uint16_t* base, int boff) {
  return *(const u32x4*)((const char*)base + boff);
}

// b128 row read that feeds MFMA A-row n of a 32-row block (physical row
// swap23(n)) with logical chunk 2c + g, i.e. k-step c of a contraction over
// the D columns (c = 0 .. D/16-1): lds_row(tile, row_off<D>(off, c)).
template <int D>
__device__ __forceinline__ void row_read_offsets(int n, int g, int* off) {
  const int r = swap23(n);
  const int h = tile_swz<D>(r);
#pragma unroll
  for (int c = 0; c < kRowOffs<D>; ++c) off[c] = (2 * (r * D + 8 * ((2 * c + g) ^ h))) & 0x7fff;
}
template <int D>
__device__ __forceinline__ int row_off(const int* off, int c) {
  return off[c % kRowOffs<D>] + 256 * (c / kRowOffs<D>);
}

// Transpose reads of 32-column block db (db = 0 .. D/32-1) for rows
// 8*(lane/32) + (lane/4)%4 of a 16-row group: lane l supplies 4 bf16 at
// logical chunk 4db + 2*((l/16)%2) + (l/2)%2, element 4*(l%2).
template <int D>
__device__ __forceinline__ void tr_read_offsets(int lane, int* off) {
  const int g = lane >> 5;
  const int r = 8 * g + ((lane >> 2) & 3);
  const int h = tile_swz<D>(r);
  const int lc = 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
#pragma unroll
  for (int db = 0; db < kTrOffs<D>; ++db)
    off[db] = (2 * (r * D + 8 * ((4 * db + lc) ^ h) + 4 * (lane & 1))) & 0x7fff;
}
template <int D>
__device__ __forceinline__ int tr_off(const int* off, int db) {
  return off[db % kTrOffs<D>] + 256 * (db / kTrOffs<D>);
}

// k-operand of a 32x32x16 MFMA contracted over 8 consecutive ROWS of a
// swizzled tile: lane l gets rows 8*(l/32) .. +7 below `rows` (a 16-row
// aligned position in the tile) of column 32*db + l%32.
template <int D>
__device__ __forceinline__ u32x4 tr_col8(const uint16_t* rows, const int* off, int db) {
  constexpr int X = D >= 128 ? 2 : 1;   // rows + 4: the swizzle's top bit flips
  const char* base = (const char*)rows;
  const u32x2 a = lds_tr4((const uint16_t*)(base + tr_off<D>(off, db)));
  const u32x2 b = lds_tr4((const uint16_t*)(base + tr_off<D>(off, db ^ X) + 8 * D));
  return u32x4{a[0], a[1], b[0], b[1]};
}

// Stores a wave's transposed accumulator X^T (lane n, g of the 32-row block:
// row n; 32-column block db: the 16 values at columns 32 db + acc_row(i, g))
// times mul (per row) as bf16 rows dst[r * D + c], r < nrows, through the
// wave's LDS region of 32 x DC bf16, DC columns per pass.  Each lane writes
// its 8-byte pieces to LDS, then reads back whole 16-byte chunks so that the
// global stores cover consecutive columns of a row: 16 lanes write 256
// contiguous bytes, where the direct stores of the accumulator layout put 8
// bytes in each of 32 rows per instruction.  Chunk k of region row r sits at
// chunk k ^ swz(r) (swz by r for 256-byte rows, r / 2 for 128-byte rows), so
// the 8-byte writes of 32 rows and the 16-byte reads of a row fall in
// distinct banks (two lanes per bank at most).
template <int D, int DC, int NDB>
__device__ __forceinline__ void store_rows_lds(uint16_t* dst, int nrows, const f32x16* acc,
                                               float mul, uint16_t* region, int lane) {
  constexpr int CPR = DC / 8;   // 16-byte chunks per region row
  static_assert(DC == 64 || DC == 128 || DC == 256, "region width");
  const int n = lane & 31, g = lane >> 5;
  auto swz = [](int r) { return DC == 64 ? (r >> 1) & 7 : r & 15; };
#pragma unroll
  for (int p = 0; p < D / DC; ++p) {
#pragma unroll
    for (int db = p * DC / 32; db < (p + 1) * DC / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int k = (db - p * DC / 32) * 4 + i4;
        const u32x2 w = {pack_bf16x2(acc[db][4 * i4] * mul, acc[db][4 * i4 + 1] * mul),
                         pack_bf16x2(acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul)};
        *(u32x2*)(region + n * DC + 8 * (k ^ swz(n)) + 4 * g) = w;
      }
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
      const int r = it * (64 / CPR) + lane / CPR, k = lane % CPR;
      const u32x4 v = *(const u32x4*)(region + r * DC + 8 * (k ^ swz(r)));
      if (r < nrows) *(u32x4*)(dst + (int64_t)r * D + p * DC + 8 * k) = v;
    }
  }
}

// An empty statement that the compiler must assume rewrites the N per-lane
// offsets in place.  At the top of a loop body it keeps the sums LDS base +
// offset inside the body, where the constant base folds into the immediate
// offset of the LDS read; otherwise they are hoisted out of the loop and each
// (base, offset) pair holds a register for the whole loop.
template <int N>
__device__ __forceinline__ void opaque_offsets(int* v) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace attn
