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
// Three kernels: per query row D and -LSE log2(e); dK and dV per key tile
// (looping over the query tiles and the query heads of a grouped key/value
// head, so every dK/dV element is written once); dQ per query tile.  No
// atomics.  Both product kernels stream their tiles HBM -> LDS with
// global_load_lds into double-buffered, swizzled tiles (see common.h) that
// are read both by rows and, through transpose reads, by columns.
#include "common.h"
#include "launch.h"

namespace attn {

// ---------------------------------------------------------------------------
// Per query row: D_i = sum_c dO[i, c] * O[i, c] and nl_i = -LSE_i * log2(e),
// both fp32, written to the workspace as [D (rows)] [nl (rows)].
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dot_do_o_kernel(const uint16_t* __restrict__ O,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ LSE,
                                                           float* __restrict__ ws, int64_t rows) {
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
  if (row < rows && sub == 0) {
    ws[row] = acc;
    ws[rows + row] = -LSE[row] * kLog2e;
  }
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
// four waves owns 32 keys, holding their K and V rows in registers (the
// B operands of S = Q K^T and dP = dO V^T) and their dK^T, dV^T accumulators.
// Query tiles of 64 rows of Q and dO, plus D and nl for those rows, stream
// through LDS.  Per 32-query sub-block, Q and dO rows are fed to the MFMA in
// swap23 order, so each lane (one key) holds P and dS for 8 contiguous
// queries per k-step: the B operands of dV^T += dO^T P and dK^T += Q^T dS,
// whose A operands dO^T and Q^T come from transpose reads of the same tiles.
// ---------------------------------------------------------------------------
template <int D>
struct BwdTile {
  static constexpr int QB = 64;   // query rows per LDS tile (dK/dV)
  static constexpr int KB = 64;   // key rows per LDS tile (dQ)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int BHk, int Hq, int Hkv, int Sq, int Skv, float scale,
    float scale_log2, int64_t rows_total) {
  constexpr int QB = BwdTile<D>::QB;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  // Double buffers as separate variables (see the forward kernel): the DMA
  // into one buffer is then known not to alias the reads of the other.
  __shared__ __attribute__((aligned(1024))) uint16_t sQ0[QB * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sQ1[QB * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sG0[QB * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sG1[QB * D];
  __shared__ __attribute__((aligned(16))) float sDn0[2 * QB];   // D then nl
  __shared__ __attribute__((aligned(16))) float sDn1[2 * QB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int bhk = blockIdx.x % BHk;
  const int ktile = blockIdx.x / BHk;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = Hq / Hkv;
  const int off = Skv - Sq;
  const int key0_wave = ktile * 128 + wave * 32;
  const int key = key0_wave + n;
  const bool kvalid = key < Skv;

  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  const float* Dd = ws;
  const float* NL = ws + rows_total;

  // Queries that can see any key of this tile: i >= first_key - off.
  const int q_begin = CAUSAL ? max(0, ktile * 128 - off) : 0;
  const int q_start = (q_begin / QB) * QB;
  const int n_qt = (Sq - q_start + QB - 1) / QB;  // query tiles per head
  const int n_it = G * n_qt;

  auto issue = [&](int it, uint16_t* dQt, uint16_t* dGt, float* dDn) {
    const int hh = it / n_qt;
    const int q0 = q_start + (it % n_qt) * QB;
    const int64_t bh = (int64_t)b * Hq + hk * G + hh;
    dma_tile<D, QB, 4>(Q + bh * Sq * D, dQt, q0, Sq, wave, lane);
    dma_tile<D, QB, 4>(dO + bh * Sq * D, dGt, q0, Sq, wave, lane);
    if (wave < 2) {
      // wave 0: D of rows q0 .. q0+63, wave 1: nl of those rows, one float
      // per lane (rows past Sq repeat row Sq-1; they are masked).
      const float* src = (wave == 0 ? Dd : NL) + bh * Sq + min(q0 + lane, Sq - 1);
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)&dDn[wave * QB],
                                       4, 0, 0);
    }
  };
  issue(0, sQ0, sG0, sDn0);

  u32x4 kreg[NDC], vreg[NDC];
  const int krow = min(key, Skv - 1);
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    kreg[c] = *(const u32x4*)(Kh + (int64_t)krow * D + c * 16 + 8 * g);
    vreg[c] = *(const u32x4*)(Vh + (int64_t)krow * D + c * 16 + 8 * g);
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkt[db][i] = dvt[db][i] = 0.f;

  int r_off[kRowOffs<D>], t_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, r_off);
  tr_read_offsets<D>(lane, t_off);

  auto step = [&](const uint16_t* cQ, const uint16_t* cG, const float* cDn, uint16_t* nQ,
                  uint16_t* nG, float* nDn, int it) {
    const int q0 = q_start + (it % n_qt) * QB;
    wait_vmcnt0();
    __syncthreads();
    if (it + 1 < n_it) issue(it + 1, nQ, nG, nDn);
#pragma unroll
    for (int sb = 0; sb < QB / 32; ++sb) {
      const int qs = q0 + sb * 32;
      // Sub-block fully hidden from this wave's keys: skip.
      if (CAUSAL && key0_wave > qs + 31 + off) continue;
      if (qs >= Sq) continue;
      // Queries past Sq read a repeated row and must not contribute; keys
      // past Skv only affect their own (unstored) dK/dV columns.
      const bool need_mask = (qs + 32 > Sq) || (CAUSAL && key0_wave + 31 > qs + off);
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      const uint16_t* qb = cQ + sb * 32 * D;
      const uint16_t* gb = cG + sb * 32 * D;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const int o = row_off<D>(r_off, c);
        s = mfma32(*(const u32x4*)(qb + o), kreg[c], s);
        dp = mfma32(*(const u32x4*)(gb + o), vreg[c], dp);
      }
      // Element i is query qs + 16*(i/8) + 8g + i%8 against key `key`.
      const float* dn = cDn + sb * 32;
      u32x4 pb[2], dsb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const f32x4 d0 = *(const f32x4*)(dn + 16 * c + 8 * g);
        const f32x4 d1 = *(const f32x4*)(dn + 16 * c + 8 * g + 4);
        const f32x4 l0 = *(const f32x4*)(dn + QB + 16 * c + 8 * g);
        const f32x4 l1 = *(const f32x4*)(dn + QB + 16 * c + 8 * g + 4);
        float pv[8], dsv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * c + j;
          const float nl = j < 4 ? l0[j] : l1[j - 4];
          const float dd = j < 4 ? d0[j] : d1[j - 4];
          float p = fast_exp2(fmaf(s[i], scale_log2, nl));
          if (need_mask) {
            const int qi = qs + 16 * c + 8 * g + j;
            const bool ok = (qi < Sq) && (!CAUSAL || key <= qi + off);
            p = ok ? p : 0.f;
          }
          pv[j] = p;
          dsv[j] = p * (dp[i] - dd);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[c][j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
          dsb[c][j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
        }
      }
      // dV^T += dO^T P,  dK^T += Q^T dS  (contracted over the 32 queries).
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvt[db] = mfma32(tr_col8<D>(gb + 16 * c * D, t_off, db), pb[c], dvt[db]);
          dkt[db] = mfma32(tr_col8<D>(qb + 16 * c * D, t_off, db), dsb[c], dkt[db]);
        }
    }
  };
#pragma clang loop unroll(disable)
  for (int it = 0; it < n_it; it += 2) {
    step(sQ0, sG0, sDn0, sQ1, sG1, sDn1, it);
    if (it + 1 < n_it) step(sQ1, sG1, sDn1, sQ0, sG0, sDn0, it + 1);
  }
  if (!kvalid) return;
  const int64_t kro = ((int64_t)(b * Hkv + hk) * Skv + key) * D;
  store_transposed<NDB>(dK + kro, dkt, g, scale);
  store_transposed<NDB>(dV + kro, dvt, g, 1.f);
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, query head, 128-query tile), 32 queries per wave
// with their Q and dO rows in registers.  Key tiles of 64 rows (K and V)
// stream through LDS.  Scores are formed transposed, S^T = K Q^T, so each
// lane (one query) holds dS^T for 8 contiguous keys per k-step: the B operand
// of dQ^T += K^T dS^T, whose A operand K^T is a transpose read of the K tile.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, uint16_t* __restrict__ dQ,
    int BH, int Hq, int Hkv, int Sq, int Skv, float scale, float scale_log2, int n_qtiles,
    int64_t rows_total) {
  constexpr int BC = BwdTile<D>::KB;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int off = Skv - Sq;
  const int wave_row0 = qtile * 128 + wave * 32;
  const int row = wave_row0 + n;
  const bool valid = row < Sq;

  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  const int last_row = min(qtile * 128 + 128, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int n_tiles = (kv_end + BC - 1) / BC;

  dma_tile<D, BC, 4>(Kh, sK0, 0, Skv, wave, lane);
  dma_tile<D, BC, 4>(Vh, sV0, 0, Skv, wave, lane);

  const int qrow = min(row, Sq - 1);
  const uint16_t* Qr = Q + ((int64_t)bh * Sq + qrow) * D;
  const uint16_t* dOr = dO + ((int64_t)bh * Sq + qrow) * D;
  u32x4 qreg[NDC], greg[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = *(const u32x4*)(Qr + c * 16 + 8 * g);
    greg[c] = *(const u32x4*)(dOr + c * 16 + 8 * g);
  }
  const float dd = ws[(int64_t)bh * Sq + qrow];
  const float nl = ws[rows_total + (int64_t)bh * Sq + qrow];
  f32x16 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqt[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;
  const int wave_kv_last = CAUSAL ? min(Skv, min(wave_row0 + 31, Sq - 1) + off + 1) - 1 : Skv - 1;
  int r_off[kRowOffs<D>], t_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, r_off);
  tr_read_offsets<D>(lane, t_off);

  auto step = [&](const uint16_t* cK, const uint16_t* cV, uint16_t* nK, uint16_t* nV, int tt) {
    const int k0 = tt * BC;
    wait_vmcnt0();
    __syncthreads();
    if (tt + 1 < n_tiles) {
      dma_tile<D, BC, 4>(Kh, nK, k0 + BC, Skv, wave, lane);
      dma_tile<D, BC, 4>(Vh, nV, k0 + BC, Skv, wave, lane);
    }
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      const int ks = k0 + kb * 32;
      if (ks > wave_kv_last) continue;
      const bool need_mask = (ks + 32 > Skv) || (CAUSAL && ks + 31 > wave_row0 + off);
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      const uint16_t* kbp = cK + kb * 32 * D;
      const uint16_t* vbp = cV + kb * 32 * D;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const int o = row_off<D>(r_off, c);
        s = mfma32(*(const u32x4*)(kbp + o), qreg[c], s);
        dp = mfma32(*(const u32x4*)(vbp + o), greg[c], dp);
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
            float p = fast_exp2(fmaf(s[i], scale_log2, nl));
            if (need_mask) {
              const int kk = ks + 16 * c + 8 * g + 2 * j + u;
              p = (kk < row_limit) ? p : 0.f;
            }
            dsv[u] = p * (dp[i] - dd);
          }
          dsb[c][j] = pack_bf16x2(dsv[0], dsv[1]);
        }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dqt[db] = mfma32(tr_col8<D>(kbp + 16 * c * D, t_off, db), dsb[c], dqt[db]);
        }
    }
  };
#pragma clang loop unroll(disable)
  for (int tt = 0; tt < n_tiles; tt += 2) {
    step(sK0, sV0, sK1, sV1, tt);
    if (tt + 1 < n_tiles) step(sK1, sV1, sK0, sV0, tt + 1);
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
                     a.stream, (const uint16_t*)a.o, (const uint16_t*)a.d_o, a.lse, a.ws, rows);
  timing_mark(a.stream, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float sl2 = a.scale * kLog2e;
  const int n_ktiles = (a.Skv + 127) / 128;
  const int BHk = a.B * a.Hkv;
  timing_mark(a.stream, 2);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(n_ktiles * BHk), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.d_o, (const float*)a.ws, (uint16_t*)a.dk, (uint16_t*)a.dv,
                     BHk, a.Hq, a.Hkv, a.Sq, a.Skv, a.scale, sl2, rows);
  timing_mark(a.stream, 3);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qtiles = (a.Sq + 127) / 128;
  const int BH = a.B * a.Hq;
  timing_mark(a.stream, 4);
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(n_qtiles * BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.d_o, (const float*)a.ws, (uint16_t*)a.dq, BH, a.Hq, a.Hkv,
                     a.Sq, a.Skv, a.scale, sl2, n_qtiles, rows);
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
