// Backward pass by recomputation.  The forward stores only O and the
// per-row log-sum-exp; every score and probability tile is rebuilt on chip
// ("Compilers and Kernels", FlashAttention section, closing paragraph: the
// backward recomputes local score and probability tiles instead of saving
// them; "Tang, a compiler that derives GPU kernels and bounds how fast they
// can run", Abstract: gradients of comprehensions are comprehensions).
//
// With P = exp(scale Q K^T + C - LSE):
//   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Three kernels: D per query row; dK and dV per key tile (looping over the
// query tiles and the query heads of a grouped key/value head, so every
// dK/dV element is written once); dQ per query tile.  No atomics.
#include "common.h"
#include "launch.h"

namespace attn {

// ---------------------------------------------------------------------------
// D_i = sum_c dO[i, c] * O[i, c] in fp32 (bf16 inputs).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_do_o_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           float* __restrict__ Dd, int64_t rows) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 o = *(const u32x4*)(O + row * D + sub * 8);
    const u32x4 g = *(const u32x4*)(dO + row * D + sub * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(__uint_as_float(o[i] << 16), __uint_as_float(g[i] << 16), acc);
      acc = fmaf(__uint_as_float(o[i] & 0xffff0000u), __uint_as_float(g[i] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int w = 1; w < LPR; w <<= 1) acc += __shfl_xor(acc, w);
  if (row < rows && sub == 0) Dd[row] = acc;
}

template <int D>
struct BwdTile {
  static constexpr int PITCH = D + 8;  // LDS row pitch in bf16
};

// 8 contiguous rows r0 .. r0+7 of column `col` of a row-major LDS tile,
// packed as 8 bf16: the k-operand of a product contracted over those rows.
__device__ __forceinline__ u32x4 bwd_col8(const uint16_t* s, int r0, int col, int pitch) {
  const uint16_t* p = s + r0 * pitch + col;
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = uint32_t(p[(2 * j) * pitch]) | (uint32_t(p[(2 * j + 1) * pitch]) << 16);
  }
  return r;
}

// Transposed accumulator X^T[d][row] (lane = row n, 16 d values per 32-d
// block) stored to row-major X[row][d] after multiplying by `mul`.
template <int NDB>
__device__ __forceinline__ void store_transposed(uint16_t* rowp, const f32x16* acc, int g,
                                                 float mul) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = db * 32 + 8 * i4 + 4 * g;
      u32x2 w = {pack_bf16x2(acc[db][4 * i4] * mul, acc[db][4 * i4 + 1] * mul),
                 pack_bf16x2(acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul)};
      *(u32x2*)(rowp + d0) = w;
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, key/value head, 128-key tile); each of its
// four waves owns 32 keys, holding their K and V rows in registers and their
// dK^T, dV^T accumulators.  Query tiles of 32 rows (Q, dO, LSE, D) are staged
// through LDS.  Scores are formed S = Q K^T with query rows fed in swap23
// order, so each lane (one key) holds P for 8 contiguous queries per k-step:
// the B operand of dV^T += dO^T P and dK^T += Q^T dS.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int Hq, int Hkv, int Sq, int Skv,
    float scale, float scale_log2, int n_ktiles) {
  constexpr int QB = 32;
  constexpr int PITCH = BwdTile<D>::PITCH;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[QB * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[QB * PITCH];
  __shared__ float sL[QB];
  __shared__ float sD[QB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int bhk = blockIdx.x % (gridDim.x / n_ktiles);
  const int ktile = blockIdx.x / (gridDim.x / n_ktiles);
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = Hq / Hkv;
  const int off = Skv - Sq;
  const int key = ktile * 128 + wave * 32 + n;
  const bool kvalid = key < Skv;

  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  u32x4 kreg[NDC], vreg[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    kreg[c] = kvalid ? *(const u32x4*)(Kh + (int64_t)key * D + c * 16 + 8 * g) : u32x4{0, 0, 0, 0};
    vreg[c] = kvalid ? *(const u32x4*)(Vh + (int64_t)key * D + c * 16 + 8 * g) : u32x4{0, 0, 0, 0};
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkt[db][i] = dvt[db][i] = 0.f;

  // Queries that can see any key of this tile: i >= first_key - off.
  const int first_key = ktile * 128;
  const int q_begin = CAUSAL ? max(0, first_key - off) : 0;
  const int q_start = (q_begin / QB) * QB;

  for (int hh = 0; hh < G; ++hh) {
    const int h = hk * G + hh;
    const int64_t bh = (int64_t)b * Hq + h;
    const uint16_t* Qh = Q + bh * Sq * D;
    const uint16_t* dOh = dO + bh * Sq * D;
    for (int q0 = q_start; q0 < Sq; q0 += QB) {
      __syncthreads();
      for (int e = tid * 8; e < QB * D; e += 256 * 8) {
        const int r = e / D, c = e % D;
        const int qi = q0 + r;
        u32x4 qx = {0, 0, 0, 0}, gx = {0, 0, 0, 0};
        if (qi < Sq) {
          qx = *(const u32x4*)(Qh + (int64_t)qi * D + c);
          gx = *(const u32x4*)(dOh + (int64_t)qi * D + c);
        }
        *(u32x4*)(sQ + r * PITCH + c) = qx;
        *(u32x4*)(sdO + r * PITCH + c) = gx;
      }
      if (tid < QB) {
        const int qi = q0 + tid;
        sL[tid] = (qi < Sq) ? LSE[bh * Sq + qi] * kLog2e : 0.f;
        sD[tid] = (qi < Sq) ? Dd[bh * Sq + qi] : 0.f;
      }
      __syncthreads();

      // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys.
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      const uint16_t* qrow = sQ + swap23(n) * PITCH + 8 * g;
      const uint16_t* grow = sdO + swap23(n) * PITCH + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        s = mfma32(*(const u32x4*)(qrow + c * 16), kreg[c], s);
        dp = mfma32(*(const u32x4*)(grow + c * 16), vreg[c], dp);
      }
      // Element i is query q0 + 16*(i/8) + 8g + i%8 against key `key`.
      u32x4 pb[2], dsb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int i = 8 * c + 2 * j + u;
            const int ql = 16 * c + 8 * g + 2 * j + u;
            const int qi = q0 + ql;
            bool ok = (qi < Sq) && kvalid;
            if (CAUSAL) ok = ok && (key <= qi + off);
            const float p = ok ? fast_exp2(s[i] * scale_log2 - sL[ql]) : 0.f;
            pv[u] = p;
            dsv[u] = p * (dp[i] - sD[ql]);
          }
          pb[c][j] = pack_bf16x2(pv[0], pv[1]);
          dsb[c][j] = pack_bf16x2(dsv[0], dsv[1]);
        }
      // dV^T += dO^T P,  dK^T += Q^T dS  (contracted over the 32 queries).
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          dvt[db] = mfma32(bwd_col8(sdO, 16 * c + 8 * g, db * 32 + n, PITCH), pb[c], dvt[db]);
          dkt[db] = mfma32(bwd_col8(sQ, 16 * c + 8 * g, db * 32 + n, PITCH), dsb[c], dkt[db]);
        }
    }
  }
  if (!kvalid) return;
  const int64_t krow = ((int64_t)(b * Hkv + hk) * Skv + key) * D;
  store_transposed<NDB>(dK + krow, dkt, g, scale);
  store_transposed<NDB>(dV + krow, dvt, g, 1.f);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, query head, 128-query tile), 32 queries per wave
// with their Q and dO rows in registers.  Key tiles of 64 rows (K and V)
// are staged in LDS.  Scores are formed transposed, S^T = K Q^T, so the lane
// (one query) holds dS^T for 8 contiguous keys per k-step: the B operand of
// dQ^T += K^T dS^T.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    uint16_t* __restrict__ dQ, int BH, int Hq, int Hkv, int Sq, int Skv, float scale,
    float scale_log2, int n_qtiles) {
  constexpr int BC = 64;
  constexpr int PITCH = BwdTile<D>::PITCH;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
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
  const int row = qtile * 128 + wave * 32 + n;
  const bool valid = row < Sq;

  const uint16_t* Qh = Q + (int64_t)bh * Sq * D;
  const uint16_t* dOh = dO + (int64_t)bh * Sq * D;
  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  u32x4 qreg[NDC], greg[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = valid ? *(const u32x4*)(Qh + (int64_t)row * D + c * 16 + 8 * g) : u32x4{0, 0, 0, 0};
    greg[c] = valid ? *(const u32x4*)(dOh + (int64_t)row * D + c * 16 + 8 * g) : u32x4{0, 0, 0, 0};
  }
  const float lse2 = valid ? LSE[(int64_t)bh * Sq + row] * kLog2e : 0.f;
  const float dd = valid ? Dd[(int64_t)bh * Sq + row] : 0.f;
  f32x16 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqt[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;
  const int last_row = min(qtile * 128 + 128, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;

  for (int k0 = 0; k0 < kv_end; k0 += BC) {
    __syncthreads();
    for (int e = tid * 8; e < BC * D; e += 256 * 8) {
      const int r = e / D, c = e % D;
      const int kk = k0 + r;
      u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
      if (kk < Skv) {
        kx = *(const u32x4*)(Kh + (int64_t)kk * D + c);
        vx = *(const u32x4*)(Vh + (int64_t)kk * D + c);
      }
      *(u32x4*)(sK + r * PITCH + c) = kx;
      *(u32x4*)(sV + r * PITCH + c) = vx;
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      const uint16_t* krow = sK + (kb * 32 + swap23(n)) * PITCH + 8 * g;
      const uint16_t* vrow = sV + (kb * 32 + swap23(n)) * PITCH + 8 * g;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        s = mfma32(*(const u32x4*)(krow + c * 16), qreg[c], s);
        dp = mfma32(*(const u32x4*)(vrow + c * 16), greg[c], dp);
      }
      u32x4 dsb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int i = 8 * c + 2 * j + u;
            const int kk = k0 + kb * 32 + 16 * c + 8 * g + 2 * j + u;
            const float p = (kk < row_limit) ? fast_exp2(s[i] * scale_log2 - lse2) : 0.f;
            dsv[u] = p * (dp[i] - dd);
          }
          dsb[c][j] = pack_bf16x2(dsv[0], dsv[1]);
        }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          dqt[db] = mfma32(bwd_col8(sK, kb * 32 + 16 * c + 8 * g, db * 32 + n, PITCH), dsb[c],
                           dqt[db]);
    }
  }
  if (!valid) return;
  store_transposed<NDB>(dQ + ((int64_t)bh * Sq + row) * D, dqt, g, scale);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  constexpr int RPB = 256 / (D / 8);
  timing_mark(a.stream, 0);
  hipLaunchKernelGGL((bwd_dot_do_o_kernel<D>), dim3((rows + RPB - 1) / RPB), dim3(256), 0,
                     a.stream, (const uint16_t*)a.o, (const uint16_t*)a.d_o, a.ws, rows);
  timing_mark(a.stream, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const int n_ktiles = (a.Skv + 127) / 128;
  timing_mark(a.stream, 2);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_ktiles * a.B * a.Hkv), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.d_o, a.lse, (const float*)a.ws, (uint16_t*)a.dk,
                     (uint16_t*)a.dv, a.Hq, a.Hkv, a.Sq, a.Skv, a.scale, sl2, n_ktiles);
  timing_mark(a.stream, 3);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qtiles = (a.Sq + 127) / 128;
  const int BH = a.B * a.Hq;
  timing_mark(a.stream, 4);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(n_qtiles * BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.d_o, a.lse, (const float*)a.ws, (uint16_t*)a.dq, BH,
                     a.Hq, a.Hkv, a.Sq, a.Skv, a.scale, sl2, n_qtiles);
  timing_mark(a.stream, 5);
  return hipGetLastError();
}

template <bool CAUSAL>
static hipError_t dispatch_bwd(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_bwd_t<64, CAUSAL>(a);
    case 128: return launch_bwd_t<128, CAUSAL>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a) {
  return a.causal ? dispatch_bwd<true>(a) : dispatch_bwd<false>(a);
}

}  // namespace attn
