// Measured ceilings of the GPU the benchmark runs on, for the roofline
// fractions it reports beside the spec peaks.  Not part of the attention
// library: built as libceilings.so and loaded only by the benchmark.
//
//   int ceil_read_run(const void* buf, int64_t bytes, void* out, int blocks, int nontemporal,
//                     void* stream)
//     grid-stride read of `bytes` (a multiple of 16) from device memory, one
//     16-byte load per thread and step, with the non-temporal hint if
//     nontemporal != 0; out: blocks * 256 uint32 (written).
//   int ceil_mfma_run(void* out, int blocks, int iters, void* stream)
//     every wave issues iters * 16 v_mfma_f32_32x32x16_bf16 on four
//     independent accumulators fed from registers (32768 FLOP each); two
//     waves per SIMD; out: blocks * 256 float (written).
// Both return the hipError_t of the launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool NT>
__global__ __launch_bounds__(256) void ceil_read(const u32x4* __restrict__ p, int64_t n16,
                                                 uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const u32x4 a = NT ? __builtin_nontemporal_load(p + i) : p[i];
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  out[blockIdx.x * 256 + threadIdx.x] = acc;
}

__device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__global__ __launch_bounds__(256, 2) void ceil_mfma(float* __restrict__ out, int iters) {
  // Small finite bf16 operands (bit patterns of values near 1/64), so the
  // accumulators stay finite.
  const u32x4 a = {0x3c803c80u, 0x3c803c80u, 0x3c803c80u, 0x3c803c80u + (threadIdx.x & 1)};
  const u32x4 b = {0x3c803c80u, 0x3c803c80u, 0x3c803c80u, 0x3c803c80u};
  f32x16 c0, c1, c2, c3;
#pragma unroll
  for (int i = 0; i < 16; ++i) c0[i] = c1[i] = c2[i] = c3[i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      c0 = mfma(a, b, c0);
      c1 = mfma(a, b, c1);
      c2 = mfma(a, b, c2);
      c3 = mfma(a, b, c3);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int ceil_read_run(const void* buf, int64_t bytes, void* out, int blocks,
                             int nontemporal, void* stream) {
  if (nontemporal)
    hipLaunchKernelGGL(ceil_read<true>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)buf, bytes / 16, (uint32_t*)out);
  else
    hipLaunchKernelGGL(ceil_read<false>, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                       (const u32x4*)buf, bytes / 16, (uint32_t*)out);
  return (int)hipGetLastError();
}

extern "C" int ceil_mfma_run(void* out, int blocks, int iters, void* stream) {
  hipLaunchKernelGGL(ceil_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, (float*)out,
                     iters);
  return (int)hipGetLastError();
}
