// Forward prefill kernels: the blockwise online-softmax recurrence
// ("Compilers and Kernels", section "FlashAttention changes the algorithm
// around IO", second display equation), one query tile per workgroup, key
// and value tiles streamed through LDS, the running (m, l, o) state of each
// query row kept in registers and O = o / l, LSE = m + ln l written once.
#include "common.h"
#include "launch.h"

namespace attn {

// ---------------------------------------------------------------------------
// float32 path: plain VALU arithmetic in fp32 end to end.
// TPR = D/32 consecutive lanes share one query row, each owning 32 of its
// columns of q and o; scores are reduced across those lanes with shuffles.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, int n_qtiles) {
  constexpr int TPR = D / 32;          // lanes per query row
  constexpr int ROWS = 256 / TPR;      // query rows per workgroup
  constexpr int BC = 32;               // keys per LDS tile
  __shared__ float sK[BC * D];
  __shared__ float sV[BC * D];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int row = qtile * ROWS + tid / TPR;
  const int col0 = (tid % TPR) * 32;
  const int off = Skv - Sq;

  const float* Qh = Q + ((int64_t)bh * Sq) * D;
  const float* Kh = K + ((int64_t)(b * Hkv + hk) * Skv) * D;
  const float* Vh = V + ((int64_t)(b * Hkv + hk) * Skv) * D;

  float q[32], o[32];
  const bool valid = row < Sq;
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    f32x4 x = valid ? *(const f32x4*)(Qh + (int64_t)row * D + col0 + c) : f32x4{0, 0, 0, 0};
    q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
    o[c] = o[c + 1] = o[c + 2] = o[c + 3] = 0.f;
  }
  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;  // keys [0, row_limit)
  const int last_row = min(qtile * ROWS + ROWS, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;

  float m = kNegInf, l = 0.f;
  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    for (int e = tid * 4; e < BC * D; e += 256 * 4) {
      const int r = e / D, c = e % D;
      const int key = k0 + r;
      f32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (key < Skv) {
        kx = *(const f32x4*)(Kh + (int64_t)key * D + c);
        vx = *(const f32x4*)(Vh + (int64_t)key * D + c);
      }
      *(f32x4*)(sK + r * D + c) = kx;
      *(f32x4*)(sV + r * D + c) = vx;
    }
    __syncthreads();

    float s[BC];
    float mx = m;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        f32x4 kx = *(const f32x4*)(sK + j * D + col0 + c);
        acc = fmaf(q[c], kx[0], acc);
        acc = fmaf(q[c + 1], kx[1], acc);
        acc = fmaf(q[c + 2], kx[2], acc);
        acc = fmaf(q[c + 3], kx[3], acc);
      }
#pragma unroll
      for (int w = 1; w < TPR; w <<= 1) acc += __shfl_xor(acc, w);
      const float x = (k0 + j < row_limit) ? acc * scale_log2 : kNegInf;
      s[j] = x;
      mx = fmaxf(mx, x);
    }
    const float msub = (mx == kNegInf) ? 0.f : mx;
    const float alpha = fast_exp2(m - msub);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < 32; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = fast_exp2(s[j] - msub);
      l += p;
#pragma unroll
      for (int c = 0; c < 32; c += 4) {
        f32x4 vx = *(const f32x4*)(sV + j * D + col0 + c);
        o[c] = fmaf(p, vx[0], o[c]);
        o[c + 1] = fmaf(p, vx[1], o[c + 1]);
        o[c + 2] = fmaf(p, vx[2], o[c + 2]);
        o[c + 3] = fmaf(p, vx[3], o[c + 3]);
      }
    }
    m = mx;
  }
  if (!valid) return;
  const float inv = 1.f / l;
  float* Oh = O + ((int64_t)bh * Sq + row) * D + col0;
#pragma unroll
  for (int c = 0; c < 32; c += 4) {
    *(f32x4*)(Oh + c) = f32x4{o[c] * inv, o[c + 1] * inv, o[c + 2] * inv, o[c + 3] * inv};
  }
  if (LSE && (tid % TPR) == 0) LSE[(int64_t)bh * Sq + row] = (m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// bf16 path: 32x32x16 bf16 MFMA with fp32 accumulation.
//
// Four waves per workgroup, 32 query rows per wave.  Scores are formed
// transposed, S^T = K Q^T (A = key rows from LDS, B = the wave's queries held
// in registers), so each lane owns ONE query column and 16 of its scores per
// 32-key block: the row maximum and row sum are lane-local plus one exchange
// with the other half-wave.  Key rows are fed to the MFMA in swap23 order so
// that the probabilities a lane holds are 8 contiguous keys, which is exactly
// the B-operand layout of O^T += V^T P^T; the accumulator O^T is again
// indexed by the lane's query, so the rescale by alpha is a per-lane scalar.
// ---------------------------------------------------------------------------
template <int D>
struct FwdTile {
  static constexpr int BC = (D >= 256) ? 32 : 64;  // keys per LDS tile
  static constexpr int PITCH = D + 8;              // LDS row pitch in bf16 (16-byte pad)
};

// V^T operand: 8 contiguous keys starting at key row `r0` of the LDS tile,
// column `col`, packed as 8 bf16.
__device__ __forceinline__ u32x4 gather_col8(const uint16_t* s, int r0, int col, int pitch) {
  const uint16_t* p = s + r0 * pitch + col;
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = uint32_t(p[(2 * j) * pitch]) | (uint32_t(p[(2 * j + 1) * pitch]) << 16);
  }
  return r;
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, int n_qtiles) {
  constexpr int BR = 128;
  constexpr int BC = FwdTile<D>::BC;
  constexpr int PITCH = FwdTile<D>::PITCH;
  constexpr int NKB = BC / 32;   // 32-key blocks per tile
  constexpr int NDC = D / 16;    // 16-wide d chunks (QK^T k-steps)
  constexpr int NDB = D / 32;    // 32-wide d blocks (PV output blocks)
  __shared__ __attribute__((aligned(16))) uint16_t sK[BC * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BC * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int off = Skv - Sq;
  const int row = qtile * BR + wave * 32 + n;
  const bool valid = row < Sq;

  const uint16_t* Qh = Q + (int64_t)bh * Sq * D;
  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;

  u32x4 qreg[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = valid ? *(const u32x4*)(Qh + (int64_t)row * D + c * 16 + 8 * g) : u32x4{0, 0, 0, 0};
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;
  const int last_row = min(qtile * BR + BR, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int first_row = qtile * BR;

  float m = kNegInf, lpart = 0.f;
  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    for (int e = tid * 8; e < BC * D; e += 256 * 8) {
      const int r = e / D, c = e % D;
      const int key = k0 + r;
      u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (key < Skv) {
        kx = *(const u32x4*)(Kh + (int64_t)key * D + c);
        vx = *(const u32x4*)(Vh + (int64_t)key * D + c);
      }
      *(u32x4*)(sK + r * PITCH + c) = kx;
      *(u32x4*)(sV + r * PITCH + c) = vx;
    }
    __syncthreads();

    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const uint16_t* krow = sK + (kb * 32 + swap23(n)) * PITCH + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        s[kb] = mfma32(*(const u32x4*)(krow + c * 16), qreg[c], s[kb]);
      }
    }
    // Keys this tile can mask: causal diagonal or the ragged end of Skv.
    const bool need_mask = (k0 + BC > Skv) || (CAUSAL && k0 + BC - 1 > first_row + off);
    float mx = m;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[kb][i] * scale_log2;
        if (need_mask) {
          const int key = k0 + kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
          if (key >= row_limit) x = kNegInf;
        }
        s[kb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor32(mx));
    const float msub = (mx == kNegInf) ? 0.f : mx;
    const float alpha = fast_exp2(m - msub);
    lpart *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    u32x4 pb[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(s[kb][8 * c + 2 * j] - msub);
          const float p1 = fast_exp2(s[kb][8 * c + 2 * j + 1] - msub);
          lpart += p0 + p1;
          pb[kb][c][j] = pack_bf16x2(p0, p1);
        }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const u32x4 a = gather_col8(sV, kb * 32 + 16 * c + 8 * g, db * 32 + n, PITCH);
          oacc[db] = mfma32(a, pb[kb][c], oacc[db]);
        }
    m = mx;
  }

  const float l = lpart + xor32(lpart);
  if (!valid) return;
  const float inv = 1.f / l;
  uint16_t* Orow = O + ((int64_t)bh * Sq + row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = db * 32 + 8 * i4 + 4 * g;
      u32x2 w = {pack_bf16x2(oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv),
                 pack_bf16x2(oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv)};
      *(u32x2*)(Orow + d0) = w;
    }
  if (LSE && g == 0) LSE[(int64_t)bh * Sq + row] = (m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const FwdArgs& a) {
  constexpr int ROWS = 256 / (D / 32);
  const int n_qtiles = (a.Sq + ROWS - 1) / ROWS;
  const int BH = a.B * a.Hq;
  timing_mark(a.stream, 0);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(n_qtiles * BH), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                     BH, a.Hq, a.Hkv, a.Sq, a.Skv, a.scale * kLog2e, n_qtiles);
  timing_mark(a.stream, 1);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
  const int n_qtiles = (a.Sq + 127) / 128;
  const int BH = a.B * a.Hq;
  timing_mark(a.stream, 0);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(n_qtiles * BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, BH, a.Hq, a.Hkv, a.Sq, a.Skv, a.scale * kLog2e,
                     n_qtiles);
  timing_mark(a.stream, 1);
  return hipGetLastError();
}

template <bool CAUSAL>
static hipError_t dispatch_fwd(const FwdArgs& a) {
  if (a.dtype == 0) {
    switch (a.d) {
      case 64: return launch_fwd_f32_t<64, CAUSAL>(a);
      case 128: return launch_fwd_f32_t<128, CAUSAL>(a);
      case 256: return launch_fwd_f32_t<256, CAUSAL>(a);
    }
  } else {
    switch (a.d) {
      case 64: return launch_fwd_bf16_t<64, CAUSAL>(a);
      case 128: return launch_fwd_bf16_t<128, CAUSAL>(a);
      case 256: return launch_fwd_bf16_t<256, CAUSAL>(a);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a) {
  return a.causal ? dispatch_fwd<true>(a) : dispatch_fwd<false>(a);
}

}  // namespace attn
