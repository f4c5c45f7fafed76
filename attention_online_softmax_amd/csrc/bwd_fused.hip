// Fused backward around the dK/dV kernel with dQ folded in (bwd.hip): the
// per-row pairs (D_i, -LSE_i log2 e) and the cleared fp32 dQ accumulator
// before it, dQ = scale * accumulator rounded to bf16 after it.  Kept apart
// from bwd.hip, whose scheduling flags do not suit these simple kernels.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace attn {

// Per padded query row r of [B * Hq, Sqp]: the pair (D_r, nl_r) exactly as
// the dQ kernel forms it ((0, -inf) for padding rows; the same products and
// order of additions, so the dK/dV kernel sees the same values).  Two
// threads per row: thread h takes the columns 16c + 8h .. 16c + 8h + 7.
// The grid also clears the n4 float4 of the dQ accumulator, grid-strided.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const uint16_t* __restrict__ O,
                                                       const uint16_t* __restrict__ dO,
                                                       const float* __restrict__ LSE,
                                                       float* __restrict__ ws,
                                                       float* __restrict__ dqacc, int64_t n4,
                                                       int64_t rows_pad, int Sq, int Sqp) {
  constexpr int NDC = D / 16;
  for (int64_t z = (int64_t)blockIdx.x * 256 + threadIdx.x; z < n4; z += (int64_t)gridDim.x * 256)
    ((f32x4*)dqacc)[z] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t r = (int64_t)blockIdx.x * 128 + (threadIdx.x >> 1);
  const int h = threadIdx.x & 1;
  if (r >= rows_pad) return;   // both threads of a row leave together
  const int64_t bh = r / Sqp;
  const int i = (int)(r - bh * Sqp);
  if (i >= Sq) {
    if (h == 0) *(f32x2*)(ws + 2 * r) = f32x2{0.f, kNegInf};
    return;
  }
  const int64_t row = bh * Sq + i;
  const uint16_t* o = O + row * D + 8 * h;
  const uint16_t* go = dO + row * D + 8 * h;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    const u32x4 x = *(const u32x4*)(o + 16 * c);
    const u32x4 y = *(const u32x4*)(go + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(x[e] << 16), __uint_as_float(y[e] << 16), acc);
      acc = fmaf(__uint_as_float(x[e] & 0xffff0000u), __uint_as_float(y[e] & 0xffff0000u), acc);
    }
  }
  acc += __shfl_xor(acc, 1);
  if (h == 0) {
    const float lse = LSE[row];
    *(f32x2*)(ws + 2 * r) = f32x2{acc, lse != kNegInf ? -lse * kLog2e : kNegInf};
  }
}

// dQ = scale * dqacc rounded to bf16, four elements per thread and step.
__global__ __launch_bounds__(256) void bwd_dq_convert_kernel(const float* __restrict__ dqacc,
                                                             uint16_t* __restrict__ dQ, int64_t n4,
                                                             float scale) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const f32x4 x = ((const f32x4*)dqacc)[i];
    ((u32x2*)dQ)[i] = u32x2{pack_bf16x2(x[0] * scale, x[1] * scale),
                            pack_bf16x2(x[2] * scale, x[3] * scale)};
  }
}

// Offset of the dQ accumulator in the fused workspace, in floats: after the
// (D, nl) pairs, rounded up to 256 bytes.
int64_t bwd_fused_acc_offset(int B, int Hq, int Sq) {
  const int64_t sqp = ((int64_t)Sq + 31) / 32 * 32;
  return (2 * (int64_t)B * Hq * sqp + 63) / 64 * 64;
}

template <int D>
static hipError_t launch_bwd_fused_t(const BwdArgs& a) {
  const int Sqp = (a.Sq + 31) / 32 * 32;
  const int64_t rows_pad = (int64_t)a.B * a.Hq * Sqp;
  float* dqacc = a.ws + bwd_fused_acc_offset(a.B, a.Hq, a.Sq);
  const int64_t n4 = (int64_t)a.B * a.Hq * a.Sq * D / 4;   // float4 of the accumulator
  ATTN_LAUNCH(0, (bwd_prep_kernel<D>), dim3((unsigned)((rows_pad + 127) / 128)), dim3(256),
              a.stream, (const uint16_t*)a.o, (const uint16_t*)a.d_o, a.lse, a.ws, dqacc,
              n4, rows_pad, a.Sq, Sqp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_dkdv_fused(a, dqacc);   // kernel 1 of the call
  if (e != hipSuccess) return e;
  // A grid of 8 workgroups per compute unit, four elements per thread and step.
  const int64_t cgrid = std::min<int64_t>((n4 + 255) / 256, 2048);
  ATTN_LAUNCH(2, bwd_dq_convert_kernel, dim3((unsigned)cgrid), dim3(256), a.stream,
              (const float*)dqacc, (uint16_t*)a.dq, n4, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_fused(const BwdArgs& a) {
  if (a.d == 64) return launch_bwd_fused_t<64>(a);
  if (a.d == 128) return launch_bwd_fused_t<128>(a);
  return hipErrorInvalidValue;
}

}  // namespace attn
