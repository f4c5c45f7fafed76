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
// 32-key block: the row maximum and row sum are lane-local plus one half-wave
// swap.  Key rows are fed to the MFMA in swap23 order so that the
// probabilities a lane holds are 8 contiguous keys, which is exactly the
// B-operand layout of O^T += V^T P^T; V^T comes straight from the row-major
// V tile through LDS transpose reads.  The accumulator O^T is again indexed
// by the lane's query, so rescaling by alpha is a per-lane scalar.
//
// K/V tiles go from HBM straight into LDS with global_load_lds (no staging
// registers), double-buffered: tile j+1 is in flight while tile j is used.
// Tiles are dense [BC][D] with 16-byte chunks XOR-swizzled per row
// (tile_swz) so that the K row reads and the V transpose reads are free of
// bank conflicts.
//
// Normalisation reference: the exponentials are taken relative to a per-row
// reference m_ref that only advances when the row maximum exceeds it by more
// than kLazy (log2 units); o and l are rescaled only then.  o, l and m_ref
// always describe the same partial softmax (o and l relative to exp2(m_ref)),
// so O = o / l and LSE = m_ref + log2 l are unchanged in exact arithmetic,
// and probabilities stay below 2^kLazy.
// ---------------------------------------------------------------------------
constexpr float kLazy = 8.f;

template <int D>
struct FwdTile {
  static constexpr int BC = 64;  // keys per LDS tile
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, (D >= 256) ? 1 : 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, int n_qtiles) {
  constexpr int BR = 128;
  constexpr int BC = FwdTile<D>::BC;
  constexpr int NKB = BC / 32;   // 32-key blocks per tile
  constexpr int NDC = D / 16;    // 16-wide d chunks (QK^T k-steps)
  constexpr int NDB = D / 32;    // 32-wide d blocks (PV output blocks)
  // Two buffers per tensor as separate variables: the compiler can then see
  // that the DMA into one buffer does not alias the reads of the other and
  // does not wait for the DMA before those reads.
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
  const int wave_row0 = qtile * BR + wave * 32;
  const int row = wave_row0 + n;
  const bool valid = row < Sq;

  const uint16_t* Qh = Q + (int64_t)bh * Sq * D;
  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;

  const int last_row = min(qtile * BR + BR, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int n_tiles = (kv_end + BC - 1) / BC;

  // Start the first tile's transfer before anything else.
  dma_tile<D, BC, 4>(Kh, sK0, 0, Skv, wave, lane);
  dma_tile<D, BC, 4>(Vh, sV0, 0, Skv, wave, lane);

  // A negative scale is applied as |scale| on -Q (bf16 negation is exact),
  // so the maximum can be taken on raw scores and scaled afterwards.
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c2 = fabsf(scale_log2);
  u32x4 qreg[NDC];
  const int qrow = min(row, Sq - 1);
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = *(const u32x4*)(Qh + (int64_t)qrow * D + c * 16 + 8 * g);
    qreg[c] ^= qsign;
  }
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;   // keys [0, row_limit)
  // Last key any row of this wave may see (tiles beyond it are skipped).
  const int wave_kv_last = CAUSAL ? min(Skv, min(wave_row0 + 31, Sq - 1) + off + 1) - 1 : Skv - 1;

  // Per-lane LDS offsets (elements) into the swizzled tiles.
  int k_off[4], v_off[2];
  row_read_offsets<D>(n, g, k_off);
  tr_read_offsets<D>(lane, v_off);

  float m_ref = kNegInf, lpart = 0.f;

  auto tile = [&](const uint16_t* cK, const uint16_t* cV, int k0, bool need_mask) {
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32(*(const u32x4*)(cK + kb * 32 * D + k_off[c & 3] + 64 * (c >> 2)),
                       qreg[c], s[kb]);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 16 * (i >> 3) + 8 * g + (i & 7);
          s[kb][i] = (key < row_limit) ? s[kb][i] : kNegInf;
        }
    }
    float rmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) rmax = fmaxf(rmax, s[kb][i]);
    const float mnew = fmaxf(m_ref, halfwave_max(rmax) * c2);
    if (__any(mnew > m_ref + kLazy)) {
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m_ref - mnew);
      lpart *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_ref = mnew;
    }
    const float msub = (m_ref == kNegInf) ? 0.f : m_ref;
    u32x4 pb[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(fmaf(s[kb][8 * c + 2 * j], c2, -msub));
          const float p1 = fast_exp2(fmaf(s[kb][8 * c + 2 * j + 1], c2, -msub));
          lpart += p0 + p1;
          pb[kb][c][j] = pack_bf16x2(p0, p1);
        }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* vp = cV + (kb * 32 + 16 * c) * D + v_off[db & 1] + 64 * (db >> 1);
          oacc[db] = mfma32(tr_col8(vp, D), pb[kb][c], oacc[db]);
        }
  };

  // One tile step: wait for tile tt, start tile tt+1 into the other buffer,
  // then use tile tt.
  auto step = [&](const uint16_t* cK, const uint16_t* cV, uint16_t* nK, uint16_t* nV, int tt) {
    const int k0 = tt * BC;
    wait_vmcnt0();      // this wave's part of tile tt has landed in LDS
    __syncthreads();    // ... and every wave's; the other buffer is free
    if (tt + 1 < n_tiles) {
      dma_tile<D, BC, 4>(Kh, nK, k0 + BC, Skv, wave, lane);
      dma_tile<D, BC, 4>(Vh, nV, k0 + BC, Skv, wave, lane);
    }
    if (k0 <= wave_kv_last) {
      const bool need_mask = (k0 + BC > Skv) || (CAUSAL && k0 + BC - 1 > wave_row0 + off);
      tile(cK, cV, k0, need_mask);
    }
  };
#pragma clang loop unroll(disable)
  for (int tt = 0; tt < n_tiles; tt += 2) {
    step(sK0, sV0, sK1, sV1, tt);
    if (tt + 1 < n_tiles) step(sK1, sV1, sK0, sV0, tt + 1);
  }

  const float l = halfwave_sum(lpart);
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
  if (LSE && g == 0) LSE[(int64_t)bh * Sq + row] = (m_ref + fast_log2(l)) * kLn2;
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
