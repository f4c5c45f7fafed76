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
// TPR consecutive lanes share one query row, each owning D/TPR of its
// columns of q and o; scores are reduced across those lanes with DPP steps.
// Large grids use 256-thread workgroups with 32 columns per lane (KW = 1:
// the four waves hold different rows and share every K/V tile).  Grids that
// would not fill the compute units use 8 columns per lane, which spreads
// the rows over 4 D/32 times as many workgroups, and KW = 8 (d <= 128, 16-key
// tiles) or 4 (d = 256): the waves of a workgroup hold the same rows and
// take every KW-th key tile each, through K/V buffers of their own, and
// their states (m, l, o) are merged by the monoid at the end.  That cuts
// the serial VALU work per row by KW.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int TPR, int NT, int KW, bool BIAS>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    int window, const float* __restrict__ bias, int64_t bsb, int64_t bsh, float scale_log2,
    int n_qtiles) {
  static_assert(KW == 1 || NT == 64 * KW, "KW > 1: one wave per key share");
  constexpr int CPL = D / TPR;         // columns per lane
  constexpr int NTR = NT / KW;         // threads that share a K/V tile
  constexpr int ROWS = NTR / TPR;      // query rows per workgroup
  constexpr int BC = (KW > 4 || (KW > 1 && D >= 256)) ? 16 : 32;   // keys per LDS tile
  __shared__ float sK[KW * BC * D];
  __shared__ float sV[KW * BC * D];

  const int tid = threadIdx.x;
  const int wk = KW > 1 ? tid / 64 : 0;     // key share of this wave
  const int ltid = KW > 1 ? tid % 64 : tid;
  float* const tK = sK + wk * BC * D;
  float* const tV = sV + wk * BC * D;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int row = qtile * ROWS + ltid / TPR;
  const int col0 = (ltid % TPR) * CPL;
  const int off = Skv - Sq;

  const float* Qh = Q + ((int64_t)bh * Sq) * D;
  const float* Kh = K + ((int64_t)(b * Hkv + hk) * Skv) * D;
  const float* Vh = V + ((int64_t)(b * Hkv + hk) * Skv) * D;

  float q[CPL];
  KahanSum o[CPL];   // compensated, like the normaliser
  const bool valid = row < Sq;
#pragma unroll
  for (int c = 0; c < CPL; c += 4) {
    f32x4 x = valid ? *(const f32x4*)(Qh + (int64_t)row * D + col0 + c) : f32x4{0, 0, 0, 0};
    q[c] = x[0]; q[c + 1] = x[1]; q[c + 2] = x[2]; q[c + 3] = x[3];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = KahanSum{0.f, 0.f};
  // Keys [row_lo, row_limit); a sliding window of `window` keys (causal
  // only, 0 = none) raises the lower end.
  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;
  const int row_lo = (CAUSAL && window > 0) ? row + off - window + 1 : 0;
  const int last_row = min(qtile * ROWS + ROWS, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int kv_begin =
      (CAUSAL && window > 0) ? max(0, qtile * ROWS + off - window + 1) / BC * BC : 0;
  // Additive bias row of this query (row i of the [Sq, Skv] bias plane); a
  // template parameter, so calls without one carry no bias loads.
  const float* brow = BIAS ? bias + b * bsb + h * bsh + (int64_t)min(row, Sq - 1) * Skv : nullptr;

  float m = kNegInf;
  KahanSum l{0.f, 0.f};
  // KW > 1: wave wk takes tiles kv_begin + wk BC, + KW BC, ...; its LDS
  // accesses are in program order, so its own buffers need no barrier.
  for (int k0 = kv_begin + wk * BC; k0 < kv_end; k0 += KW * BC) {
    if (KW == 1) __syncthreads();
    // The tile in groups of up to 8 16-byte chunks per lane and tensor, all
    // loads of a group issued before its LDS stores (one memory round trip
    // per group, not per chunk).
    constexpr int NCH = BC * D / (NTR * 4);   // chunks per lane and tensor
    constexpr int GRP = NCH < 8 ? NCH : 8;
#pragma unroll
    for (int i0 = 0; i0 < NCH; i0 += GRP) {
      f32x4 kx[GRP], vx[GRP];
#pragma unroll
      for (int i = 0; i < GRP; ++i) {
        // Rows past the last key load the last row and are zeroed after
        // (no branch around the loads).
        const int e = ((i0 + i) * NTR + ltid) * 4;
        const int key = k0 + e / D, c = e % D;
        const int64_t kr = (int64_t)min(key, Skv - 1) * D + c;
        kx[i] = *(const f32x4*)(Kh + kr);
        vx[i] = *(const f32x4*)(Vh + kr);
      }
#pragma unroll
      for (int i = 0; i < GRP; ++i) {
        const int e = ((i0 + i) * NTR + ltid) * 4;
        const bool in = k0 + e / D < Skv;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        *(f32x4*)(tK + e) = in ? kx[i] : zero;
        *(f32x4*)(tV + e) = in ? vx[i] : zero;
      }
    }
    if (KW == 1) __syncthreads();

    float s[BC];
    float mx = m;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        f32x4 kx = *(const f32x4*)(tK + j * D + col0 + c);
        acc = fmaf(q[c], kx[0], acc);
        acc = fmaf(q[c + 1], kx[1], acc);
        acc = fmaf(q[c + 2], kx[2], acc);
        acc = fmaf(q[c + 3], kx[3], acc);
      }
      acc = group_reduce<TPR, false>(acc);
      float x = acc * scale_log2;
      if constexpr (BIAS) x = fmaf(brow[min(k0 + j, Skv - 1)], kLog2e, x);
      s[j] = (k0 + j < row_limit && k0 + j >= row_lo) ? x : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float msub = (mx == kNegInf) ? 0.f : mx;
    const float alpha = fast_exp2(m - msub);
    // The tile's terms are summed from zero, then added to the rescaled
    // running (l, o): one by one, terms far below a large running value
    // would round away over long sequences.
    float lt = 0.f, ot[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) ot[c] = 0.f;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = fast_exp2(s[j] - msub);
      lt += p;
#pragma unroll
      for (int c = 0; c < CPL; c += 4) {
        f32x4 vx = *(const f32x4*)(tV + j * D + col0 + c);
        ot[c] = fmaf(p, vx[0], ot[c]);
        ot[c + 1] = fmaf(p, vx[1], ot[c + 1]);
        ot[c + 2] = fmaf(p, vx[2], ot[c + 2]);
        ot[c + 3] = fmaf(p, vx[3], ot[c + 3]);
      }
    }
    l.scale(alpha);
    l.add(lt);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      o[c].scale(alpha);
      o[c].add(ot[c]);
    }
    m = mx;
  }
  if constexpr (KW > 1) {
    // Merge the KW states of each lane (same row and columns in every
    // wave) in wave order: M = max m_w, weights 2^(m_w - M) (0 for a wave
    // that saw no key), l and o summed with those weights.
    constexpr int NV = CPL + 2;
    __syncthreads();   // every wave has left its tile loop
    if (wk > 0) {
      sK[((wk - 1) * NV + 0) * 64 + ltid] = m;
      sK[((wk - 1) * NV + 1) * 64 + ltid] = l.value();
#pragma unroll
      for (int c = 0; c < CPL; ++c) sK[((wk - 1) * NV + 2 + c) * 64 + ltid] = o[c].value();
    }
    __syncthreads();
    if (wk > 0) return;
    float M = m;
#pragma unroll
    for (int w = 1; w < KW; ++w) M = fmaxf(M, sK[((w - 1) * NV) * 64 + ltid]);
    const float f0 = m == kNegInf ? 0.f : fast_exp2(m - M);
    float lm = l.value() * f0, om[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) om[c] = o[c].value() * f0;
#pragma unroll
    for (int w = 1; w < KW; ++w) {
      const float mw = sK[((w - 1) * NV) * 64 + ltid];
      const float fw = mw == kNegInf ? 0.f : fast_exp2(mw - M);
      lm = fmaf(sK[((w - 1) * NV + 1) * 64 + ltid], fw, lm);
#pragma unroll
      for (int c = 0; c < CPL; ++c) om[c] = fmaf(sK[((w - 1) * NV + 2 + c) * 64 + ltid], fw, om[c]);
    }
    m = M;
    l = KahanSum{lm, 0.f};
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = KahanSum{om[c], 0.f};
  }
  if (!valid) return;
  const float lv = l.value();
  const float inv = lv > 0.f ? 1.f / lv : 0.f;   // a row with no allowed key: O = 0, LSE = -inf
  float* Oh = O + ((int64_t)bh * Sq + row) * D + col0;
#pragma unroll
  for (int c = 0; c < CPL; c += 4) {
    *(f32x4*)(Oh + c) = f32x4{o[c].value() * inv, o[c + 1].value() * inv,
                              o[c + 2].value() * inv, o[c + 3].value() * inv};
  }
  if (LSE && (ltid % TPR) == 0) LSE[(int64_t)bh * Sq + row] = (m + fast_log2(lv)) * kLn2;
}

// ---------------------------------------------------------------------------
// bf16 path: 32x32x16 bf16 MFMA with fp32 accumulation.
//
// NW (2, 4 or 8, chosen per call) waves per workgroup, 32 query rows per
// wave; the waves share every K/V tile.  Scores are formed
// transposed, S^T = K Q^T (A = key rows from LDS, B = the wave's queries held
// in registers), so each lane owns ONE query column and 16 of its scores per
// 32-key block: the row maximum and row sum are lane-local plus one half-wave
// swap.  Key rows are fed to the MFMA in swap23 order so that the
// probabilities a lane holds are 8 contiguous keys, which is exactly the
// B-operand layout of O^T += V^T P^T; V^T comes straight from the row-major
// V tile through LDS transpose reads.  The accumulator O^T is again indexed
// by the lane's query, so rescaling by alpha is a per-lane scalar.
//
// K/V tiles of BC keys (32 or 64, chosen per call) go from HBM straight
// into LDS with buffer loads to LDS (no staging registers), double-buffered:
// tile j+1 is requested when tile j's loop body starts.  Tiles are dense
// [BC][D] with 16-byte chunks XOR-swizzled per row (tile_swz) so that the K
// row reads and the V transpose reads are free of bank conflicts.
//
// Normalisation reference: the exponentials are taken relative to a per-row
// reference m_ref that only advances when a tile's probabilities against it
// would reach 2^kLazy (detected from their sum, so the common tile needs no
// row maximum); o and l are rescaled only then.  o, l and m_ref always
// describe the same partial softmax (o and l relative to exp2(m_ref)), so
// O = o / l and LSE = m_ref + log2 l are unchanged in exact arithmetic, and
// probabilities stay below 2^kLazy.
// ---------------------------------------------------------------------------
constexpr float kLazy = 8.f;
constexpr float kLazyBound = 256.f;   // 2^kLazy

// Keys per K/V tile (BC, 32 or 64) and waves per workgroup (NW, 32 query
// rows each) are template parameters; the launcher picks them per call from
// a per-tile time estimate (fwd_tiles.cpp).  The bias path adds its values
// tile by tile for 32 keys.  Two waves per SIMD must fit (at most 256
// registers), except for the eight-wave d256 kernel, which is the only
// workgroup on its compute unit, and the d256 bias kernel, whose bias
// values need registers beyond 256 (one wave per SIMD, up to 512).
template <int D, int NW, bool BIAS>
constexpr int kFwdMinWaves = (D >= 256 && (NW == 8 || BIAS)) ? 1 : 2;

// SPLIT = 2: the workgroup's waves form two groups of NW/2, each with the
// same NW/2 32-row query blocks; group h takes the key tiles j0 + h,
// j0 + h + 2, ... (each group loads its own tiles), and the second group's
// (m, l, o) of every row is merged into the first's at the end by the
// online-softmax monoid ("Tang, a compiler that derives GPU kernels and
// bounds how fast they can run", Abstract).  A causal grid with few query
// tiles per compute unit then takes half the key steps per workgroup.
template <int D, bool CAUSAL, int NW, int BC, bool WIN, bool BIAS, int SPLIT = 1>
__global__ __launch_bounds__(64 * NW, (kFwdMinWaves<D, NW, BIAS>)) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    int window, const float* __restrict__ bias, int64_t bsb, int64_t bsh, float scale_log2,
    int n_qtiles) {
  static_assert(!BIAS || BC == 32, "the bias path works on 32-key tiles");
  static_assert(SPLIT == 1 || (SPLIT == 2 && NW == 4 && BC >= 32 && !WIN && !BIAS),
                "key halves: two groups of two waves, plain calls");
  constexpr int NQ = NW / SPLIT; // 32-row query blocks per workgroup
  constexpr int BR = 32 * NQ;    // query rows per workgroup
  constexpr int NKB = BC / 32;   // 32-key blocks per tile
  constexpr int NDC = D / 16;    // 16-wide d chunks (QK^T k-steps)
  constexpr int NDB = D / 32;    // 32-wide d blocks (PV output blocks)
  // Two tile buffers per tensor, as separate variables: the compiler can
  // then see which buffer each transfer writes and each read reads, and
  // does not wait for the transfer into one before reading the other.
  // With SPLIT = 2 each buffer holds one tile per key group.
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[SPLIT * BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[SPLIT * BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[SPLIT * BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[SPLIT * BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  // Work item: query tile t (heaviest first when causal) of key/value head
  // hk of batch b, ranked r = t * B * Hkv + b * Hkv + hk, and one of its G
  // query heads.  Workgroup ids congruent mod 8 run on the same XCD, so the
  // G query heads of item r take ids 8 (G (r / 8) + j) + r % 8, j < G: they
  // read the item's key/value tiles through one L2.
  const int G = Hq / Hkv;
  const int BHk = BH / G;   // B * Hkv
  const int qq = blockIdx.x >> 3;
  const int r = (qq / G) * 8 + (blockIdx.x & 7);
  if (r >= n_qtiles * BHk) return;   // padding of the last group of 8 items
  const int t = r / BHk;
  const int b = (r % BHk) / Hkv, hk = (r % BHk) % Hkv;
  const int h = hk * G + qq % G;
  const int bh = b * Hq + h;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int off = Skv - Sq;
  const int q0 = qtile * BR;
  const int qb = SPLIT == 1 ? wave : wave % NQ;   // the wave's 32-row block
  const int kg = SPLIT == 1 ? 0 : wave / NQ;      // its key group
  const int kgo = kg * BC * D;                    // its tiles' offset in a buffer
  const int row = q0 + qb * 32 + n;
  const bool valid = row < Sq;

  const uint16_t* Qh = Q + (int64_t)bh * Sq * D;
  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  TileDma<D, BC, NQ> dma;   // a key group's tile, moved by its NQ waves
  dma.init(qb, lane);

  const int last_row = min(q0 + BR, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int n_tiles = (kv_end + BC - 1) / BC;
  // A sliding window of `window` keys (causal only, 0 = none): row i sees
  // keys [i + off - window + 1, i + off].  The loop starts at the first tile
  // the workgroup's first row can see; tiles below t_lo cut some row's
  // lower bound and are masked too.
  const bool win = WIN;   // instantiated for causal calls with window > 0 only
  const int j0 = win ? max(0, q0 + off - window + 1) / BC : 0;
  const int t_lo = win ? max(0, last_row + off - window + 1 + BC - 1) / BC : 0;
  // Tiles from t_mask on cut some row's causal bound.
  int t_mask = Skv / BC;
  if (CAUSAL) t_mask = min(t_mask, (q0 + off + 1) / BC);

  // A negative scale is applied as |scale| on -Q (bf16 negation is exact),
  // so the maximum can be taken on raw scores and scaled afterwards.  A zero
  // scale makes every score 0: Q is replaced by zeros and the scale by 1,
  // which gives the same exact scores while masked ones stay -inf (a raw
  // -inf times a zero scale would be NaN).
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = scale_log2 == 0.f ? 0u : 0xffffffffu;
  const float c2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);
  // With an additive bias the scores are taken to the log2 domain before the
  // softmax (s c2 + bias log2(e)), which then works with unit scale.
  const float c2s = BIAS ? 1.f : c2;
  u32x4 qreg[NDC];
  const int qrow = min(row, Sq - 1);
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = *(const u32x4*)(Qh + (int64_t)qrow * D + c * 16 + 8 * g);
    qreg[c] = (qreg[c] ^ qsign) & qkeep;
  }
  dma.load(Kh, Skv, sK0 + kgo, (j0 + kg) * BC, qb);
  dma.load(Vh, Skv, sV0 + kgo, (j0 + kg) * BC, qb);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;   // keys [row_lo, row_limit)
  const int row_lo = win ? row + off - window + 1 : 0;

  // Per-lane LDS byte offsets into the swizzled tiles.
  int k_off[kRowOffs<D>], v_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, k_off);
  tr_read_offsets<D>(lane, v_off);

  float m_ref = kNegInf;
  KahanSum lpart{0.f, 0.f};

  // S^T(tile) = K(tile) Q^T for this wave's 32 queries.
  auto qk = [&](const uint16_t* cK, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        s[kb] = mfma32(lds_row(cK + kb * 32 * D, row_off<D>(k_off, c)), qreg[c], s[kb]);
    // Keep three K reads in flight ahead of the products; left alone, the
    // scheduler issues each read right before its product at this register
    // pressure and every product waits for the LDS latency.
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);   // 3 LDS reads
#pragma unroll
    for (int i = 0; i < NDC * NKB - 3; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  };
  // Scores of keys outside [row_lo, row_limit) become -inf.
  auto mask = [&](f32x16* s, int k0) {
    const int lim = row_limit - k0 - 8 * g;
    const int lo = row_lo - k0 - 8 * g;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = kb * 32 + 16 * (i >> 3) + (i & 7);
        s[kb][i] = (kk < lim && kk >= lo) ? s[kb][i] : kNegInf;
      }
  };
  // One tile of the online softmax: advance the reference if the tile's
  // maximum passes it by more than kLazy, fold the tile's exponentials into
  // lpart and pack them as the B operand of the PV product.  Returns the
  // factor by which o must be rescaled (1 unless the reference moved).
  auto softmax = [&](const f32x16* s, u32x4 (*pb)[2]) {
    // Fast path: exponentials against the current reference.  A lane's sum
    // below 2^kLazy bounds each of its probabilities by 2^kLazy, the same
    // bound the lazy reference keeps, so no row maximum is needed.  A larger
    // sum, inf or NaN (e.g. m_ref still -inf on the first tile) takes the
    // slow path: advance the reference to the row maximum, rescale, redo.
    auto exps = [&](float msub) {
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float p0 = fast_exp2(fmaf(s[kb][8 * c + 2 * j], c2s, -msub));
            const float p1 = fast_exp2(fmaf(s[kb][8 * c + 2 * j + 1], c2s, -msub));
            sum += p0 + p1;
            pb[kb][c][j] = pack_bf16x2(p0, p1);
          }
      return sum;
    };
    float lsum = exps(m_ref);
    float alpha = 1.f;
    if (__any(!(lsum < kLazyBound))) {
      float rmax = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) rmax = fmaxf(rmax, s[kb][i]);
      const float mnew = fmaxf(m_ref, halfwave_max(rmax) * c2s);
      alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m_ref - mnew);
      m_ref = mnew;
      lsum = exps((m_ref == kNegInf) ? 0.f : m_ref);
    }
    lpart.scale(alpha);
    lpart.add(lsum);
    return alpha;
  };


  // O^T += V(tile)^T P^T.
  auto pv = [&](const uint16_t* cV, const u32x4 (*pb)[2]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          oacc[db] = mfma32(tr_col8<D>(cV + (kb * 32 + 16 * c) * D, v_off, db), pb[kb][c],
                            oacc[db]);
        }
  };

  {
    // Tile loop: wait for tile j, start tile j+1 into the other buffers,
    // then S(j), softmax, O += P(j) V(j).  Two or more waves per SIMD (the
    // register budget of every head dimension allows it) overlap the matrix
    // products of one wave with the softmax and LDS latency of another.
    // Tiles past the last key of this wave's rows are skipped.
    const int wave_kv_last =
        CAUSAL ? min(Skv, min(q0 + qb * 32 + 31, Sq - 1) + off + 1) - 1 : Skv - 1;
    const int wave_kv_first = win ? q0 + qb * 32 + off - window + 1 : 0;
    // Additive bias of this lane's query for the keys it holds: keys
    // k0 + 16c + 8g + 0..7 (c = 0, 1) in bv[2c], bv[2c + 1].  The next
    // tile's values are requested while the current tile is used.
    const float* brow =
        BIAS ? bias + b * bsb + h * bsh + (int64_t)min(row, Sq - 1) * Skv : nullptr;
    auto load_bias = [&](int k0, f32x4* bv) {
      if (k0 + BC <= Skv) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = *(const f32x4*)(brow + k0 + 16 * (e >> 1) + 8 * g + 4 * (e & 1));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int x = 0; x < 4; ++x)
            bv[e][x] = brow[min(k0 + 16 * (e >> 1) + 8 * g + 4 * (e & 1) + x, Skv - 1)];
      }
    };
    f32x4 bnext[4];
    if constexpr (BIAS) load_bias(j0 * BC, bnext);
    f32x16 s[NKB];
    u32x4 p[NKB][2];
    // Step j0 + SPLIT i: this wave's tile is j = the step's first tile plus
    // its key group (past n_tiles for the second group of an odd count:
    // skipped below, as tiles past the wave's keys are).
    auto step = [&](int j, const uint16_t* cK, const uint16_t* cV, uint16_t* nK, uint16_t* nV) {
      j += kg;
      cK += kgo;
      cV += kgo;
      wait_vmcnt0();   // this wave's part of tile j has landed
      lds_barrier();   // ... and every wave's; tile j-1 is no longer read
      opaque_offsets<kRowOffs<D>>(k_off);
      opaque_offsets<kTrOffs<D>>(v_off);
      dma.load(Kh, Skv, nK + kgo, (j + SPLIT) * BC, qb);
      dma.load(Vh, Skv, nV + kgo, (j + SPLIT) * BC, qb);
      f32x4 bcur[4];
      if constexpr (BIAS) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bcur[e] = bnext[e];
        if (j + 1 < n_tiles) load_bias((j + 1) * BC, bnext);
      }
      if (j * BC > wave_kv_last || j * BC + BC - 1 < wave_kv_first) return;
      qk(cK, s);
      if constexpr (BIAS) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          s[0][i] = fmaf(s[0][i], c2, bcur[2 * (i >> 3) + ((i & 7) >> 2)][i & 3] * kLog2e);
      }
      if (j >= t_mask || j < t_lo) mask(s, j * BC);
      const float alpha = softmax(s, p);
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      pv(cV, p);
    };
#pragma clang loop unroll(disable)
    for (int j = j0; j < n_tiles; j += 2 * SPLIT) {
      step(j, sK0, sV0, sK1, sV1);
      if (j + SPLIT < n_tiles) step(j + SPLIT, sK1, sV1, sK0, sV0);
    }
  }

  float l = halfwave_sum(lpart.value());
  if constexpr (SPLIT == 2) {
    // The second key group parks its (m, l, o) in LDS at its lanes'
    // positions; the first folds it into its own state (same rows, same
    // lane layout) and alone stores O and LSE.  o of block qb: buffer sK0
    // or sV0; m and l: past the O staging area of sK1 or sV1.
    wait_vmcnt0();   // the transfer issued by the last step (past the keys) has landed
    lds_barrier();
    float* mo = (float*)(qb == 0 ? sK0 : sV0);
    float* ml = (float*)((qb == 0 ? sK1 : sV1) + 32 * D);
    if (kg == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) mo[(db * 16 + i) * 64 + lane] = oacc[db][i];
      ml[lane] = m_ref;
      ml[64 + lane] = l;
    }
    lds_barrier();
    if (kg == 1) return;   // past the workgroup's last barrier
    const float m1 = ml[lane], l1 = ml[64 + lane];
    const float M = fmaxf(m_ref, m1);
    const float w0 = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - M);
    const float w1 = m1 == kNegInf ? 0.f : fast_exp2(m1 - M);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = fmaf(w1, mo[(db * 16 + i) * 64 + lane], w0 * oacc[db][i]);
    l = fmaf(w1, l1, w0 * l);
    m_ref = M;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;   // a row with no allowed key: O = 0, LSE = -inf
  if (LSE && g == 0 && valid) LSE[(int64_t)bh * Sq + row] = (m_ref + fast_log2(l)) * kLn2;
  if constexpr (SPLIT == 2) {
    // O of block qb through the first 32 rows of sK1 or sV1.
    store_rows_lds<D, D, NDB>(O + ((int64_t)bh * Sq + q0 + qb * 32) * D,
                              min(32, Sq - (q0 + qb * 32)), oacc, inv, qb == 0 ? sK1 : sV1, lane);
    return;
  }
  // O through LDS (the tile buffers, free once every wave is past the last
  // tile): wave w's region of 32 rows x DC columns.
  constexpr int DC = (BC * D / (8 * NW)) < D ? BC * D / (8 * NW) : D;
  constexpr int PER = BC * D / (32 * DC);   // regions per tile buffer
  static_assert(PER >= 1 && NW <= 4 * PER, "O staging must fit the tile buffers");
  wait_vmcnt0();   // the transfer issued by the last step (past the keys) has landed
  lds_barrier();
  const int a = wave / PER;
  uint16_t* region = (a == 0 ? sK0 : a == 1 ? sK1 : a == 2 ? sV0 : sV1) + (wave % PER) * 32 * DC;
  store_rows_lds<D, DC, NDB>(O + ((int64_t)bh * Sq + q0 + wave * 32) * D,
                             min(32, Sq - (q0 + wave * 32)), oacc, inv, region, lane);
}

// ---------------------------------------------------------------------------
// bf16 key-split forward, for grids with few query blocks per compute unit.
//
// A workgroup of NW waves takes ONE 32-row query block, and its waves split
// the block's 32-key tiles: wave w takes tiles w, w + NW, w + 2 NW, ...,
// each wave with its own online-softmax state (m, l, o).  The NW states of
// every row are then merged through LDS with the monoid operation ("Tang, a
// compiler that derives GPU kernels and bounds how fast they can run",
// Abstract: online softmax as a monoid; the same merge as the split-KV
// decode).  A heavy causal query block then takes about
// 1/NW of its key tiles in time instead of all of them.
//
// No tile is shared between waves, so there is no barrier in the loop.  Key
// rows go from HBM straight into the MFMA A-operand registers (the wave's
// next tile is requested when the current one starts); V tiles go through a
// per-wave double buffer in LDS, for the transpose reads.  Scores, softmax
// and P V are those of fwd_bf16_kernel for one wave and one 32-key block.
// ---------------------------------------------------------------------------
// One 32-key block of the online softmax with the lazy reference of
// fwd_bf16_kernel: the block's exponentials against m_ref, packed as the B
// operand of the P V product; the reference moves (and the returned factor
// differs from 1) only when they would reach 2^kLazy.
__device__ __forceinline__ float softmax_block(const f32x16& s, u32x4 (&pb)[2], float& m_ref,
                                               KahanSum& lpart, float c2) {
  auto exps = [&](float msub) __attribute__((always_inline)) {
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(s[8 * c + 2 * j], c2, -msub));
        const float p1 = fast_exp2(fmaf(s[8 * c + 2 * j + 1], c2, -msub));
        sum += p0 + p1;
        pb[c][j] = pack_bf16x2(p0, p1);
      }
    return sum;
  };
  float lsum = exps(m_ref);
  float alpha = 1.f;
  if (__any(!(lsum < kLazyBound))) {
    float rmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) rmax = fmaxf(rmax, s[i]);
    const float mnew = fmaxf(m_ref, halfwave_max(rmax) * c2);
    alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m_ref - mnew);
    m_ref = mnew;
    lsum = exps((m_ref == kNegInf) ? 0.f : m_ref);
  }
  lpart.scale(alpha);
  lpart.add(lsum);
  return alpha;
}

// Taken only where the grid has at most one query block per compute unit,
// so two waves per SIMD are plenty (no register cap below 256).
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_ks_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int Hq, int Hkv, int Sq, int Skv,
    float scale_log2, int n_qtiles) {
  constexpr int BC = 32;
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int VBUF = BC * D;   // one V tile, bf16 elements
  // Per-wave V buffers, as two arrays (distinct objects: the compiler sees
  // which buffer a transfer writes and a read reads).  After the loop they
  // hold the waves' o rows for the merge: rows 0-15 of wave w in sV0's part
  // of wave w, rows 16-31 in sV1's (16 rows x D floats = one V tile).
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[NW * VBUF];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[NW * VBUF];
  __shared__ float sML[NW * 32 * 2];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  // Work item and XCD grouping as in fwd_bf16_kernel.
  const int G = Hq / Hkv;
  const int BHk = BH / G;
  const int qq = blockIdx.x >> 3;
  const int r = (qq / G) * 8 + (blockIdx.x & 7);
  if (r >= n_qtiles * BHk) return;
  const int t = r / BHk;
  const int b = (r % BHk) / Hkv, hk = (r % BHk) % Hkv;
  const int h = hk * G + qq % G;
  const int bh = b * Hq + h;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int off = Skv - Sq;
  const int q0 = qtile * 32;
  const int row = q0 + n;

  const uint16_t* Qh = Q + (int64_t)bh * Sq * D;
  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  const int last_row = min(q0 + 32, Sq) - 1;
  const int kv_end = CAUSAL ? max(0, min(Skv, last_row + off + 1)) : Skv;
  const int n_tiles = (kv_end + BC - 1) / BC;
  int t_mask = Skv / BC;   // tiles from t_mask on cut some row's key range
  if (CAUSAL) t_mask = min(t_mask, (q0 + off + 1) / BC);

  // Scale sign and zero scale as in fwd_bf16_kernel.
  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = scale_log2 == 0.f ? 0u : 0xffffffffu;
  const float c2 = scale_log2 == 0.f ? 1.f : fabsf(scale_log2);
  u32x4 qreg[NDC];
  const int qrow = min(row, Sq - 1);
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = *(const u32x4*)(Qh + (int64_t)qrow * D + c * 16 + 8 * g);
    qreg[c] = (qreg[c] ^ qsign) & qkeep;
  }

  // Key rows: lane (n, g) holds row swap23(n) of the tile, columns
  // 8 (2c + g) .. +7 for k-step c, loaded through a buffer resource over the
  // whole [Skv, D] matrix (rows past Skv read as zeros).
  const rsrc_t rk = make_rsrc(Kh, (uint32_t)Skv * D * 2);
  const int kvoff = (swap23(n) * D + 8 * g) * 2;
  auto load_k = [&](int j, u32x4* kr) __attribute__((always_inline)) {
    const int soff = (int)((uint32_t)j * BC * D * 2);
#pragma unroll
    for (int c = 0; c < NDC; ++c) kr[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, kvoff + 32 * c, soff, 0);
  };
  TileDma<D, BC, 1> dma;
  dma.init(0, lane);
  uint16_t* v0 = sV0 + wave * VBUF;
  uint16_t* v1 = sV1 + wave * VBUF;
  int v_off[kTrOffs<D>];
  tr_read_offsets<D>(lane, v_off);

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_ref = kNegInf;
  KahanSum lpart{0.f, 0.f};
  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;

  u32x4 kA[NDC], kB[NDC];
  auto step = [&](int j, const u32x4* kc, u32x4* kn, const uint16_t* cV, uint16_t* nV)
      __attribute__((always_inline)) {
    wait_vmcnt0();   // tile j's key rows and V tile have landed
    opaque_offsets<kTrOffs<D>>(v_off);
    if (j + NW < n_tiles) {
      load_k(j + NW, kn);
      dma.load(Vh, Skv, nV, (j + NW) * BC, 0);
    }
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c) s = mfma32(kc[c], qreg[c], s);
    if (j >= t_mask) {
      const int lim = row_limit - j * BC - 8 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 16 * (i >> 3) + (i & 7);
        s[i] = kk < lim ? s[i] : kNegInf;
      }
    }
    u32x4 p[2];
    const float alpha = softmax_block(s, p, m_ref, lpart, c2);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(tr_col8<D>(cV + 16 * c * D, v_off, db), p[c], oacc[db]);
  };
  if (wave < n_tiles) {
    load_k(wave, kA);
    dma.load(Vh, Skv, v0, wave * BC, 0);
  }
#pragma clang loop unroll(disable)
  for (int j = wave; j < n_tiles; j += 2 * NW) {
    step(j, kA, kB, v0, v1);
    if (j + NW < n_tiles) step(j + NW, kB, kA, v1, v0);
  }

  // Merge.  Each wave parks (m, l) and its o rows in LDS (o columns XOR-
  // swizzled by the row so that rows at one column fall in distinct banks);
  // then wave w combines columns [w D/NW, (w+1) D/NW) of all 32 rows.
  const float l = halfwave_sum(lpart.value());
  __syncthreads();   // every wave is done with its V buffers
  const int sw = (n & 15) << 2;
  {
    float* ob = (float*)(n < 16 ? v0 : v1) + (n & 15) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = db * 32 + 8 * i4 + 4 * g;
        *(f32x4*)(ob + (col ^ sw)) = f32x4{oacc[db][4 * i4], oacc[db][4 * i4 + 1],
                                           oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]};
      }
    if (g == 0) {
      sML[(wave * 32 + n) * 2] = m_ref;
      sML[(wave * 32 + n) * 2 + 1] = l;
    }
  }
  __syncthreads();
  constexpr int CL = D / NW / 2;   // output columns per lane
  float mw[NW], wt[NW];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mw[w] = sML[(w * 32 + n) * 2];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    wt[w] = mw[w] == kNegInf ? 0.f : fast_exp2(mw[w] - M);
    L += wt[w] * sML[(w * 32 + n) * 2 + 1];
  }
  const int c0 = wave * (D / NW) + g * CL;
  float acc[CL];
#pragma unroll
  for (int k = 0; k < CL; ++k) acc[k] = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const float* ob = (const float*)(n < 16 ? sV0 : sV1) + w * VBUF / 2 + (n & 15) * D;
#pragma unroll
    for (int k = 0; k < CL; k += 4) {
      const f32x4 x = *(const f32x4*)(ob + ((c0 + k) ^ sw));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[k + e] = fmaf(wt[w], x[e], acc[k + e]);
    }
  }
  if (row >= Sq) return;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint16_t* Orow = O + ((int64_t)bh * Sq + row) * D + c0;
#pragma unroll
  for (int k = 0; k < CL; k += 8) {
    u32x4 w = {pack_bf16x2(acc[k] * inv, acc[k + 1] * inv), pack_bf16x2(acc[k + 2] * inv, acc[k + 3] * inv),
               pack_bf16x2(acc[k + 4] * inv, acc[k + 5] * inv), pack_bf16x2(acc[k + 6] * inv, acc[k + 7] * inv)};
    *(u32x4*)(Orow + k) = w;
  }
  if (LSE && wave == 0 && g == 0) LSE[(int64_t)bh * Sq + row] = (M + fast_log2(L)) * kLn2;
}

// ---------------------------------------------------------------------------
// Host launchers.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, int TPR, int NT, int KW, bool BIAS>
static hipError_t launch_fwd_f32_k(const FwdArgs& a) {
  constexpr int ROWS = NT / KW / TPR;
  const int n_qtiles = (a.Sq + ROWS - 1) / ROWS;
  const int BH = a.B * a.Hq;
  ATTN_LAUNCH(0, (fwd_f32_kernel<D, CAUSAL, TPR, NT, KW, BIAS>), dim3(n_qtiles * BH), dim3(NT),
              a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o,
              a.lse, BH, a.Hq, a.Hkv, a.Sq, a.Skv, a.window, a.bias, a.bias_sb, a.bias_sh,
              a.scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int TPR, int NT, int KW>
static hipError_t launch_fwd_f32_c(const FwdArgs& a) {
  if (a.bias) return launch_fwd_f32_k<D, CAUSAL, TPR, NT, KW, true>(a);
  return launch_fwd_f32_k<D, CAUSAL, TPR, NT, KW, false>(a);
}

// Fewer 256-thread workgroups than compute units: 8 columns per lane and
// the keys split over the waves of each workgroup.
template <int D, bool CAUSAL>
static hipError_t launch_fwd_f32_t(const FwdArgs& a) {
  constexpr int ROWS = 256 / (D / 32);
  const int64_t big = (int64_t)((a.Sq + ROWS - 1) / ROWS) * a.B * a.Hq;
  if (big < device_cus()) {
    // d <= 128: eight waves of 16-key tiles (their K/V buffers fit in LDS);
    // d = 256: four waves.
    if constexpr (D <= 128)
      return launch_fwd_f32_c<D, CAUSAL, D / 8, 512, 8>(a);
    else
      return launch_fwd_f32_c<D, CAUSAL, D / 8, 256, 4>(a);
  }
  return launch_fwd_f32_c<D, CAUSAL, D / 32, 256, 1>(a);
}

// One bf16 forward launch with NW waves per workgroup and BC keys per tile.
template <int D, bool CAUSAL, int NW, int BC, bool WIN, bool BIAS, int SPLIT = 1>
static hipError_t launch_fwd_bf16_k(const FwdArgs& a) {
  constexpr int BR = 32 * NW / SPLIT;   // query rows per workgroup
  const int n_qtiles = (a.Sq + BR - 1) / BR;
  const int BH = a.B * a.Hq;
  // Items of (query tile, batch, key/value head) in groups of 8, one
  // workgroup per query head of each (see the kernel's work mapping).
  const int items = n_qtiles * a.B * a.Hkv;
  const int grid = (items + 7) / 8 * 8 * (a.Hq / a.Hkv);
  ATTN_LAUNCH(0, (fwd_bf16_kernel<D, CAUSAL, NW, BC, WIN, BIAS, SPLIT>), dim3(grid),
              dim3(64 * NW), a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
              (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, BH, a.Hq, a.Hkv, a.Sq, a.Skv,
              a.window, a.bias, a.bias_sb, a.bias_sh, a.scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

// Candidate (NW, BC) of the plain (no window, no bias) kernel: launch it, or
// with fn != nullptr only report its function (for occupancy queries).
template <int D, bool CAUSAL, int NW, int BC, int SPLIT = 1>
static hipError_t fwd_candidate(const FwdArgs* a, const void** fn) {
  if (fn) {
    *fn = reinterpret_cast<const void*>(&fwd_bf16_kernel<D, CAUSAL, NW, BC, false, false, SPLIT>);
    return hipSuccess;
  }
  return launch_fwd_bf16_k<D, CAUSAL, NW, BC, false, false, SPLIT>(*a);
}

// Key-split candidate: NW waves per 32-row query block.
template <int D, bool CAUSAL, int NW>
static hipError_t fwd_candidate_ks(const FwdArgs* a, const void** fn) {
  if (fn) {
    *fn = reinterpret_cast<const void*>(&fwd_bf16_ks_kernel<D, CAUSAL, NW>);
    return hipSuccess;
  }
  const int n_qtiles = (a->Sq + 31) / 32;
  const int items = n_qtiles * a->B * a->Hkv;
  const int grid = (items + 7) / 8 * 8 * (a->Hq / a->Hkv);
  ATTN_LAUNCH(0, (fwd_bf16_ks_kernel<D, CAUSAL, NW>), dim3(grid), dim3(64 * NW), a->stream,
              (const uint16_t*)a->q, (const uint16_t*)a->k, (const uint16_t*)a->v,
              (uint16_t*)a->o, a->lse, a->B * a->Hq, a->Hq, a->Hkv, a->Sq, a->Skv,
              a->scale * kLog2e, n_qtiles);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t fwd_candidate_i(int idx, const FwdArgs* a, const void** fn) {
  // Must list the candidates of fwd_tile_candidates() in the same order.
  if constexpr (D == 64) {
    switch (idx) {
      case 0: return fwd_candidate<D, CAUSAL, 4, 64>(a, fn);
      case 1: return fwd_candidate<D, CAUSAL, 4, 32>(a, fn);
      case 2: return fwd_candidate<D, CAUSAL, 8, 64>(a, fn);
      case 3: return fwd_candidate<D, CAUSAL, 2, 64>(a, fn);
      case 4: return fwd_candidate_ks<D, CAUSAL, 4>(a, fn);
      case 5: return fwd_candidate_ks<D, CAUSAL, 2>(a, fn);
      case 6: return fwd_candidate<D, CAUSAL, 4, 64, 2>(a, fn);
    }
  } else if constexpr (D == 128) {
    switch (idx) {
      case 0: return fwd_candidate<D, CAUSAL, 4, 32>(a, fn);
      case 1: return fwd_candidate<D, CAUSAL, 4, 64>(a, fn);
      case 2: return fwd_candidate<D, CAUSAL, 8, 32>(a, fn);
      case 3: return fwd_candidate<D, CAUSAL, 8, 64>(a, fn);
      case 4: return fwd_candidate_ks<D, CAUSAL, 4>(a, fn);
      case 5: return fwd_candidate_ks<D, CAUSAL, 2>(a, fn);
      case 6: return fwd_candidate<D, CAUSAL, 4, 32, 2>(a, fn);
    }
  } else {
    switch (idx) {
      case 0: return fwd_candidate<D, CAUSAL, 8, 32>(a, fn);
      case 1: return fwd_candidate<D, CAUSAL, 4, 32>(a, fn);
    }
  }
  return hipErrorInvalidValue;
}

// Function of candidate idx of the plain bf16 forward (d, causal).
hipError_t fwd_candidate_fn(int d, bool causal, int idx, const void** fn) {
  switch (d) {
    case 64: return causal ? fwd_candidate_i<64, true>(idx, nullptr, fn)
                           : fwd_candidate_i<64, false>(idx, nullptr, fn);
    case 128: return causal ? fwd_candidate_i<128, true>(idx, nullptr, fn)
                            : fwd_candidate_i<128, false>(idx, nullptr, fn);
    case 256: return causal ? fwd_candidate_i<256, true>(idx, nullptr, fn)
                            : fwd_candidate_i<256, false>(idx, nullptr, fn);
  }
  return hipErrorInvalidValue;
}

// The sliding window and the additive bias are template parameters: calls
// without them run the kernel with none of their arithmetic.  Plain calls
// take the candidate the tile estimate picks; windowed or biased calls a
// fixed shape (the bias path: 32-key tiles).
template <int D, bool CAUSAL, bool WIN, bool BIAS>
static hipError_t launch_fwd_bf16_w(const FwdArgs& a) {
  if constexpr (!WIN && !BIAS) {
    const int idx = fwd_pick_candidate(a);
    return fwd_candidate_i<D, CAUSAL>(idx, &a, nullptr);
  } else {
    // d256 with a bias: four waves at one per SIMD (the bias values of a
    // tile need registers beyond the eight-wave kernel's 256).
    constexpr int NW = (D >= 256 && !BIAS) ? 8 : 4;
    constexpr int BC = (D == 64 && !BIAS) ? 64 : 32;
    return launch_fwd_bf16_k<D, CAUSAL, NW, BC, WIN, BIAS>(a);
  }
}

// An additive bias is a template parameter too.
template <int D, bool CAUSAL, bool WIN>
static hipError_t launch_fwd_bf16_b(const FwdArgs& a) {
  if (a.bias) return launch_fwd_bf16_w<D, CAUSAL, WIN, true>(a);
  return launch_fwd_bf16_w<D, CAUSAL, WIN, false>(a);
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
  if constexpr (CAUSAL) {
    if (a.window > 0) return launch_fwd_bf16_b<D, true, true>(a);
  }
  return launch_fwd_bf16_b<D, CAUSAL, false>(a);
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
