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
// Two kernels: dQ per query tile, which also forms D and -LSE log2(e) per
// query row and passes them on through the workspace; then dK and dV per key
// tile (looping over the query tiles and the query heads of a grouped
// key/value head, so every dK/dV element is written once).  No atomics.  Both
// product kernels stream their tiles HBM -> LDS with loads to LDS into
// double-buffered, swizzled tiles (see common.h) that are read both by rows
// and, through transpose reads, by columns.
//
// The fused variant runs the dK/dV kernel once with dQ folded in: each key
// tile adds its share dS K to an fp32 dQ accumulator with atomic adds, so the
// order of the additions, and with it the last bits of dQ, can change from
// run to run.  A small kernel forms the (D, -LSE log2(e)) pairs and clears the
// accumulator before it, another scales and rounds dQ to bf16 after it.
#pragma once

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace attn {

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

// The same for a float32 destination (partial sums): 16 bytes per store.
template <int NDB>
__device__ __forceinline__ void store_transposed_f32(float* rowp, const f32x16* acc, int g,
                                                     float mul) {
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = db * 32 + 8 * i4 + 4 * g;
      *(f32x4*)(rowp + d0) = f32x4{acc[db][4 * i4] * mul, acc[db][4 * i4 + 1] * mul,
                                   acc[db][4 * i4 + 2] * mul, acc[db][4 * i4 + 3] * mul};
    }
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (b, key/value head, 128-key tile); each of its
// four waves owns 32 keys and their dK^T, dV^T accumulators.  The K rows of
// the wave's keys are held in registers (B operand of S = Q K^T); the V rows
// of the workgroup's 128 keys sit in LDS for the whole kernel (B operand of
// dP = dO V^T, read by rows), which keeps a wave within the 256 registers of
// two waves per SIMD.  Query tiles of 32 rows of Q and dO, plus D and nl of
// those rows, are double-buffered through LDS (rows past Sq arrive as zeros
// and have nl = -inf).  Q and dO rows are fed to the MFMA in swap23 order, so
// each lane (one key) holds P and dS for 8 contiguous queries per k-step:
// the B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands dO^T
// and Q^T come from transpose reads of the same tiles.  The loop covers the
// query tiles of all query heads of the group.
//
// FUSED: the K and V roles swap (K rows of the workgroup in LDS, the lane's
// V row in registers), and after every query tile the waves stage dS (bf16,
// [query][key]) in LDS; wave w then forms columns 32 (w % (d/32)) .. +31 of
// dQ_tile = dS K over its share of the 128 keys (all of them for d = 128,
// half for d = 64), with K from transpose reads of the K rows, and adds the
// result to the fp32 accumulator dqacc [B, Hq, Sq, d] with atomic adds.
// ---------------------------------------------------------------------------
// Two waves per SIMD (at most 256 registers) up to d = 128; at d = 256 the
// dK and dV accumulators alone take 256 registers per lane, so one wave per
// SIMD (up to 512).
template <int D>
constexpr int kBwdMinWaves = D >= 256 ? 1 : 2;

// The fused dK/dV kernel at d = 128: its dQ products (and a window's or a
// bias's state) do not fit 256 registers next to the dK and dV
// accumulators (it spilled 8 to 175 registers), so it runs at one wave per
// SIMD with the accumulation registers as well.  On B4 H16 S2048: window
// 512 with a bias 496 -> 365 us, the bias alone 671 -> 574 us, causal 541
// -> 520 us.  The two-kernel dK/dV kernel with a window and a bias keeps two
// waves per SIMD and its 8-register spill: at one wave it was 13 % slower.
template <int D, bool FUSED>
constexpr int kBwdDkdvMinWaves = (FUSED && D == 128) ? 1 : kBwdMinWaves<D>;

// Small grids (fewer 128-key workgroups than compute units, e.g. grouped
// heads with few key/value heads): NKW 32-key blocks per workgroup and HS
// groups of NKW waves.  Group h takes every HS-th iteration (query head,
// query tile) of the loop, h, h + HS, ..., with Q/dO slots of its own, and at
// the end groups 1 .. HS-1 add their dK/dV sums into group 0's through LDS.
// (NKW, HS) = (4, 1) is the plain kernel; (4, 2) and (2, 4) run eight waves,
// two per SIMD, on the same number of keys or half of them.
//
// PS (head split, plain calls only): the G query heads of a key/value head
// are dealt over `hsplit` workgroups per key tile (workgroup p takes heads
// p, p + hsplit, ...), each of which writes its float32 sums of dK (times
// scale) and dV to part[p][0 | 1][B, Hkv, Skv, d]; bwd_dkdv_reduce_kernel
// adds the partials and rounds them to dK and dV.
template <int D, bool CAUSAL, bool WIN, bool BIAS, bool FUSED, int NKW = 4, int HS = 1,
          bool PS = false>
__global__ __launch_bounds__(64 * NKW * HS, (kBwdDkdvMinWaves<D, FUSED>)) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ ws, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int BHk, int Hq, int Hkv, int Sq, int Sqp, int Skv, int window,
    const float* __restrict__ bias, int64_t bsb, int64_t bsh, float scale, float scale_log2,
    int64_t rows_pad, int diag, float* __restrict__ dqacc, int hsplit,
    float* __restrict__ part) {
  static_assert((NKW == 4 && HS == 1) || (!FUSED && D <= 128 && NKW * HS == 8 &&
                                          (HS - 1) * NKW <= 2 * HS),
                "(4, 1), or eight waves of a plain kernel at d <= 128");
  static_assert(!PS || (!FUSED && !WIN && !BIAS), "head split: plain calls only");
  constexpr int NW = NKW * HS;   // waves per workgroup
  constexpr int KT = 32 * NKW;   // keys per workgroup
  constexpr int QT = 32;   // query rows per tile
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  // Slot: Q tile, dO tile, then D and nl of its rows (2 x QT floats).  One
  // variable per slot (and for V): the compiler tracks transfers into LDS
  // per variable and so never waits for the transfer into one slot before
  // reading another.
  constexpr int SLOT = 2 * QT * D + 4 * QT;
  // dS staging (FUSED): 32 query rows of 128 keys, padded so that both the
  // column writes and the row reads are free of bank conflicts.
  constexpr int SSTR = 128 + 8;
  __shared__ __attribute__((aligned(1024))) uint16_t sT0[HS * SLOT];   // one slot per group
  __shared__ __attribute__((aligned(1024))) uint16_t sT1[HS * SLOT];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[KT * D];   // K rows when FUSED
  __shared__ __attribute__((aligned(16))) uint16_t sS[FUSED ? QT * SSTR : 8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int kbw = HS == 1 ? wave : wave % NKW;   // the wave's key block, and its index in the group
  const int hg = HS == 1 ? 0 : wave / NKW;       // its group
  const int n = lane & 31, g = lane >> 5;
  const int pidx = PS ? (int)(blockIdx.x % (unsigned)hsplit) : 0;   // head split share
  const int wg = PS ? (int)(blockIdx.x / (unsigned)hsplit) : (int)blockIdx.x;
  const int bhk = wg % BHk;
  const int ktile = wg / BHk;
  const int b = bhk / Hkv, hk = bhk % Hkv;
  const int G = Hq / Hkv;
  // Query heads of this workgroup: all G, or (PS) G / hsplit of them; head
  // index hh of the loop is query head hk G + head(hh).
  const int Gl = PS ? (G - pidx + hsplit - 1) / hsplit : G;
  auto head = [&](int hh) { return PS ? pidx + hsplit * hh : hh; };
  const int off = diag;   // key j is visible to query i iff j <= i + off (causal)
  const int key0_wave = ktile * KT + kbw * 32;
  // Lane n owns key swap23(n) of the wave's 32: the V rows it needs as the
  // B operand of dP are then read exactly like the Q and dO rows.
  const int key = key0_wave + swap23(n);
  const bool kvalid = key < Skv;

  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;

  // Queries that can see any key of this tile: i >= first_key - off, and
  // with a sliding window of `window` keys (causal only, 0 = none) also
  // i < last_key - off + window.
  const bool win = WIN;   // instantiated for causal calls with window > 0 only
  const int q_start = CAUSAL ? (max(0, ktile * KT - off) / QT) * QT : 0;
  const int q_end = win ? min(Sq, ktile * KT + KT - 1 - off + window) : Sq;
  // Query tiles per head; 0 when no query's window reaches these keys
  // (possible only with a window and Sq < Skv).
  const int n_qt = max(0, (q_end - q_start + QT - 1) / QT);
  const int n_it = Gl * n_qt;

  // The workgroup's V rows, K rows when FUSED (rows past Skv arrive as zeros).
  {
    TileDma<D, KT, NW> vdma;
    vdma.init(wave, lane);
    vdma.load(FUSED ? Kh : Vh, Skv, sV, ktile * KT, wave);
  }
  TileDma<D, QT, NKW> dma;   // the group's tiles, moved by its NKW waves
  dma.init(kbw, lane);
  // The (D, nl) pairs of a tile's 32 rows: 256 contiguous bytes, one float
  // per lane of wave 0, through a descriptor over the whole workspace
  // (< 4 GiB).
  const rsrc_t ws_rs = make_rsrc(ws, (uint32_t)(2 * rows_pad * 4));
  // Transfer of the group's next iteration tile (query head dma_hh, query
  // tile dma_qt) into its part of `slot`; past the last tile nothing is
  // fetched.  Iterations advance by HS: (hh, qt) moves HS tiles on.
  auto advance = [&](int& hh, int& qt, int by) {
    qt += by;
    while (qt >= n_qt && hh < Gl) {   // at most HS passes (n_qt >= 1 when it matters)
      qt -= n_qt;
      ++hh;
    }
  };
  int dma_hh = 0, dma_qt = 0;
  if constexpr (HS > 1) {
    if (n_qt > 0) advance(dma_hh, dma_qt, hg);
    else dma_hh = Gl;
  }
  auto issue = [&](uint16_t* slot0) {
    if (dma_hh >= Gl) return;
    uint16_t* slot = slot0 + hg * SLOT;
    const int q0 = q_start + dma_qt * QT;
    const int64_t bh = (int64_t)b * Hq + hk * G + head(dma_hh);
    if (kbw == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ws_rs, (__attribute__((address_space(3))) void*)(slot + 2 * QT * D), 4, lane * 4,
          (int)((uint32_t)(bh * Sqp + q0) * 8), 0, 0);
    dma.load(Q + bh * Sq * D, Sq, slot, q0, kbw);
    dma.load(dO + bh * Sq * D, Sq, slot + QT * D, q0, kbw);
    if constexpr (HS == 1) {
      if (++dma_qt == n_qt) {
        dma_qt = 0;
        ++dma_hh;
      }
    } else {
      advance(dma_hh, dma_qt, HS);
    }
  };
  issue(sT0);

  // The lane's K row (V row when FUSED).
  u32x4 kreg[NDC];
  const int krow = min(key, Skv - 1);
  const uint16_t* Rh = FUSED ? Vh : Kh;
#pragma unroll
  for (int c = 0; c < NDC; ++c) kreg[c] = *(const u32x4*)(Rh + (int64_t)krow * D + c * 16 + 8 * g);

  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dkt[db][i] = dvt[db][i] = 0.f;

  int r_off[kRowOffs<D>], t_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, r_off);
  tr_read_offsets<D>(lane, t_off);
  const uint16_t* sVw = sV + kbw * 32 * D;

  // One tile: S = Q K^T and dP = dO V^T (element i: query 16*(i/8) + 8g +
  // i%8 of the tile, key `key`); P = exp(scale S - LSE), dS = P (dP - D);
  // dV^T += dO^T P, dK^T += Q^T dS.  Only the softmax step is inside the
  // mask branch; the accumulators are updated outside it.
  // Additive bias of this lane's key for the tile's queries (element (c, j)
  // is query qs + 16c + 8g + j), requested before the products that precede
  // its use.
  const int bkey = min(key, Skv - 1);
  auto load_bias = [&](int qs, int hh, float* bv) {
    const float* bp = bias + b * bsb + (int64_t)(hk * G + hh) * bsh + bkey;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      bv[i] = bp[(int64_t)min(qs + 16 * (i >> 3) + 8 * g + (i & 7), Sq - 1) * Skv];
  };
  // FUSED: dS of the lane's key for queries 16c + 8g + 0..7 into column
  // `kl` of the staging rows.
  const int kl = wave * 32 + swap23(n);
  auto stage_ds = [&](int c, const u32x4& v) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sS[(16 * c + 8 * g + j) * SSTR + kl] = (uint16_t)(v[j >> 1] >> (16 * (j & 1)));
  };
  auto step = [&](const uint16_t* slot, int qs, int hh) {
    const uint16_t* cQ = slot;
    const uint16_t* cG = slot + QT * D;
    const float* cN = (const float*)(slot + 2 * QT * D);
    float bv[16];
    if constexpr (BIAS) load_bias(qs, hh, bv);
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c) {
      const int o = row_off<D>(r_off, c);
      s = mfma32(lds_row(cQ, o), FUSED ? lds_row(sVw, o) : kreg[c], s);
      dp = mfma32(lds_row(cG, o), FUSED ? kreg[c] : lds_row(sVw, o), dp);
    }
    // The softmax step and the products in two halves of 16 queries, so only
    // half of P and dS is live at a time.  FUSED also masks keys past Skv,
    // whose dS would otherwise enter dQ.
    const bool masked = (CAUSAL && key0_wave + 31 > qs + off) ||
                        (win && key0_wave < qs + QT + off - window) ||
                        (FUSED && key0_wave + 31 >= Skv);
    // Element (c, j) is query qs + 16c + 8g + j: visible iff lo <= 16c + j
    // (causal) and 16c + j <= hi (window).
    const int lo = key - off - qs - 8 * g;
    const int hi = win ? lo + window - 1 : 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 pb, dsb;
      auto softmax = [&](auto msk) {
        // (D, nl) of queries 16c + 8g + 0..7
        f32x4 dn[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) dn[k] = *(const f32x4*)(cN + 2 * (16 * c + 8 * g) + 4 * k);
        float pv[8], dsv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * c + j;
          const float dd = dn[j >> 1][2 * (j & 1)];
          const float nl = dn[j >> 1][2 * (j & 1) + 1];
          float p = fast_exp2(fmaf(s[i], scale_log2, BIAS ? fmaf(bv[i], kLog2e, nl) : nl));
          if constexpr (decltype(msk)::value)
            p = ((!CAUSAL || 16 * c + j >= lo) && 16 * c + j <= hi && (!FUSED || kvalid)) ? p
                                                                                      : 0.f;
          pv[j] = p;
          dsv[j] = p * (dp[i] - dd);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pb[j] = pack_bf16x2(pv[2 * j], pv[2 * j + 1]);
          dsb[j] = pack_bf16x2(dsv[2 * j], dsv[2 * j + 1]);
        }
      };
      if (masked)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      if constexpr (FUSED) stage_ds(c, dsb);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvt[db] = mfma32(tr_col8<D>(cG + 16 * c * D, t_off, db), pb, dvt[db]);
        dkt[db] = mfma32(tr_col8<D>(cQ + 16 * c * D, t_off, db), dsb, dkt[db]);
      }
    }
  };

  // FUSED: dQ[qs .. qs+31, 32 qdb .. +31] += dS[:, kb0 .. kb0+KW-1] K[kb0 .., :]
  // for query head hh; element i of lane (n, g) is query 8(i/4) + 4g + i%4,
  // column 32 qdb + n, so each atomic instruction covers 128 contiguous bytes
  // of two rows.  The atomics go through one descriptor per 8-row group of
  // the tile, over the group's rows below Sq: rows past Sq fall outside its
  // range and are dropped (the offsets are per-lane and immediate, both of
  // which the range check covers).
  constexpr int KW = 128 * NDB / 4;   // keys per wave in the dQ product
  const int qdb = wave % NDB, kb0 = (wave / NDB) * KW;
  const int dq_voff = (4 * g * D + qdb * 32 + n) * 4;
  auto dq_tile = [&](int qs, int hh) {
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
    for (int c = 0; c < KW / 16; ++c) {
      const int kr = kb0 + 16 * c;
      // Keys of a wave that skipped this tile have no dS staged (the skip
      // test of the loop body, for the wave that owns keys kr).
      const int kw0 = ktile * 128 + (kr & ~31);
      if (CAUSAL && qs + QT - 1 + off < kw0) continue;
      if (win && qs + off - window + 1 > kw0 + 31) continue;
      const u32x4 a = *(const u32x4*)(sS + n * SSTR + kr + 8 * g);
      acc = mfma32(a, tr_col8<D>(sV + kr * D, t_off, qdb), acc);
    }
    // Reads of step c + 1 while step c multiplies: a short lookahead keeps
    // the registers of this phase within the budget of two waves per SIMD.
#pragma unroll
    for (int c = 0; c < KW / 16; ++c) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      if (c > 0) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    const float* tile = dqacc + ((int64_t)(b * Hq + hk * G + hh) * Sq + qs) * D;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const rsrc_t rs = make_rsrc(tile + 8 * gq * D, (uint32_t)(max(0, min(Sq - qs - 8 * gq, 8)) * D * 4));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[4 * gq + r], rs, dq_voff + r * D * 4,
                                                        0, 0);
    }
  };

  int cur_qt = 0, cur_hh = 0;   // query tile and query head of the group's next step
  if constexpr (HS > 1) {
    if (n_qt > 0) advance(cur_hh, cur_qt, hg);
    else cur_hh = Gl;
  }
  auto body = [&](const uint16_t* cur0, uint16_t* nxt) {
    wait_vmcnt0();   // this wave's part of the current tile (and V) has landed
    lds_barrier();   // ... and every wave's; the other slot is no longer read
    opaque_offsets<kRowOffs<D>>(r_off);
    opaque_offsets<kTrOffs<D>>(t_off);
    issue(nxt);
    const uint16_t* cur = cur0 + hg * SLOT;
    const int qs = q_start + cur_qt * QT;
    const int hh = head(cur_hh);
    if constexpr (HS == 1) {
      if (++cur_qt == n_qt) {
        cur_qt = 0;
        ++cur_hh;
      }
    } else {
      if (cur_hh >= Gl) return;   // the group has no iteration left (the last step)
      advance(cur_hh, cur_qt, HS);
    }
    // Tiles whose queries all precede this wave's first visible key, or
    // whose windows all start after its last key: skip (FUSED: the dQ
    // product leaves out the keys of waves that skip).
    const bool skip = (CAUSAL && qs + QT - 1 + off < key0_wave) ||
                      (win && qs + off - window + 1 > key0_wave + 31);
    if (!skip) step(cur, qs, hh);
    if constexpr (FUSED) {
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's dS writes are done
      lds_barrier();                        // ... and every wave's
      dq_tile(qs, hh);
    }
  };
  const int n_steps = (n_it + HS - 1) / HS;   // steps of every group (the last may be idle)
#pragma clang loop unroll(disable)
  for (int i = 0; i < n_steps; i += 2) {
    body(sT0, sT1);
    if (i + 1 < n_steps) body(sT1, sT0);
  }
  wait_vmcnt0();   // nothing in flight into LDS when the workgroup ends (n_it may be 0)
  if constexpr (HS > 1) {
    // Groups 1 .. HS-1 add their sums into group 0's: one half of the
    // columns of one accumulator per round, group h's partial of the wave
    // with key block kb at red[((h - 1) NKW + kb) 32 D / 2 + ...] (floats),
    // laid out by lane so that writes and reads are plain 16-byte rows.
    float* red = reinterpret_cast<float*>(sT0);
    constexpr int HALF = NDB / 2 > 0 ? NDB / 2 : 1;   // accumulator blocks per round
    constexpr int ROUNDS = NDB / HALF;
#pragma unroll
    for (int acc = 0; acc < 2; ++acc)
#pragma unroll
      for (int rd = 0; rd < ROUNDS; ++rd) {
        lds_barrier();   // the slots (and the previous round) are no longer read
        f32x16* A = acc == 0 ? dvt : dkt;
        if (hg > 0) {
          float* dst = red + ((hg - 1) * NKW + kbw) * (HALF * 16 * 64) + lane * 4;
#pragma unroll
          for (int e = 0; e < HALF; ++e)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
              *(f32x4*)(dst + (e * 4 + i4) * 256) =
                  f32x4{A[rd * HALF + e][4 * i4], A[rd * HALF + e][4 * i4 + 1],
                        A[rd * HALF + e][4 * i4 + 2], A[rd * HALF + e][4 * i4 + 3]};
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's writes are done
        lds_barrier();
        if (hg == 0) {
#pragma unroll
          for (int h = 1; h < HS; ++h) {
            const float* src = red + ((h - 1) * NKW + kbw) * (HALF * 16 * 64) + lane * 4;
#pragma unroll
            for (int e = 0; e < HALF; ++e)
#pragma unroll
              for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 v = *(const f32x4*)(src + (e * 4 + i4) * 256);
#pragma unroll
                for (int j = 0; j < 4; ++j) A[rd * HALF + e][4 * i4 + j] += v[j];
              }
          }
        }
      }
    if (hg > 0) return;
  }
  if (!kvalid) return;
  const int64_t kro = ((int64_t)(b * Hkv + hk) * Skv + key) * D;
  if constexpr (PS) {
    const int64_t nkv = (int64_t)BHk * Skv * D;
    store_transposed_f32<NDB>(part + 2 * pidx * nkv + kro, dkt, g, scale);
    store_transposed_f32<NDB>(part + (2 * pidx + 1) * nkv + kro, dvt, g, 1.f);
  } else {
    store_transposed<NDB>(dK + kro, dkt, g, scale);
    store_transposed<NDB>(dV + kro, dvt, g, 1.f);
  }
}

// dK and dV of the head split: the sum of the hsplit partials, in order,
// rounded to bf16.  Eight elements per thread and step.  (A template on the
// head dimension only so that each source including this header names its
// own instantiation.)
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_reduce_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ dK,
                                                              uint16_t* __restrict__ dV,
                                                              int64_t nkv, int hsplit) {
  const int64_t n8 = nkv / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n8;
       i += (int64_t)gridDim.x * 256) {
    const int t = i >= n8;   // 0: dK, 1: dV
    const int64_t e = (i - t * n8) * 8;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, c = {0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < hsplit; ++p) {
      const float* src = part + (2 * p + t) * nkv + e;
      const f32x4 x = *(const f32x4*)src, y = *(const f32x4*)(src + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a[j] += x[j];
        c[j] += y[j];
      }
    }
    const u32x4 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(c[0], c[1]),
                     pack_bf16x2(c[2], c[3])};
    *(u32x4*)((t ? dV : dK) + e) = w;
  }
}

template <int D>
struct BwdTile {
  // key rows per LDS tile (dQ): four buffers of KB x D bf16 (64 KB at d256)
  static constexpr int KB = D >= 256 ? 32 : 64;
};

// ---------------------------------------------------------------------------
// dQ: one workgroup per (b, query head, 128-query tile), 32 queries per wave
// with their Q and dO rows in registers.  It runs first and also forms, per
// query row, D_i = sum_c dO[i, c] O[i, c] and nl_i = -LSE_i * log2(e),
// which it uses itself and writes to the workspace as pairs (D_i, nl_i) for
// the dK/dV kernel; each head's rows are padded to Sqp = Sq rounded up to
// 32 and the padding rows get (0, -inf), so their probabilities are exactly
// 0 there.  Key tiles (K and V) are
// double-buffered through LDS by buffer loads.  Scores are formed transposed, S^T = K Q^T, so each
// lane (one query) holds dS^T for 8 contiguous keys per k-step: the B operand
// of dQ^T += K^T dS^T, whose A operand K^T is a transpose read of the K tile.
// ---------------------------------------------------------------------------
//
// Small grids: NQW 32-row query blocks per workgroup and HS groups of NQW
// waves (as in the dK/dV kernel); group h takes the key tiles t0 + h,
// t0 + h + HS, ... through buffers of its own, and groups 1 .. HS-1 add
// their dQ sums into group 0's through LDS at the end.  (4, 1) is the plain
// kernel; the eight-wave shapes (4, 2) and (2, 4) use 32-key tiles.
template <int D, bool CAUSAL, bool WIN, bool BIAS, int NQW = 4, int HS = 1>
__global__ __launch_bounds__(64 * NQW * HS, (kBwdMinWaves<D>)) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const uint16_t* __restrict__ O,
    const float* __restrict__ LSE, float* __restrict__ ws, uint16_t* __restrict__ dQ, int BH,
    int Hq, int Hkv, int Sq, int Sqp, int Skv, int window, const float* __restrict__ bias,
    int64_t bsb, int64_t bsh, float scale, float scale_log2, int n_qtiles) {
  static_assert((NQW == 4 && HS == 1) || (D <= 128 && NQW * HS == 8),
                "(4, 1), or eight waves at d <= 128");
  constexpr int BC = HS == 1 ? BwdTile<D>::KB : 32;
  constexpr int BR = 32 * NQW;   // query rows per workgroup
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[HS * BC * D];   // one tile per group
  __shared__ __attribute__((aligned(1024))) uint16_t sK1[HS * BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[HS * BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV1[HS * BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int qb = HS == 1 ? wave : wave % NQW;   // the wave's 32-row block, and its index in the group
  const int hg = HS == 1 ? 0 : wave / NQW;      // its group
  const int go = hg * BC * D;                   // the group's tile in each buffer
  const int n = lane & 31, g = lane >> 5;
  const int bh = blockIdx.x % BH;
  const int t = blockIdx.x / BH;
  const int qtile = CAUSAL ? (n_qtiles - 1 - t) : t;
  const int b = bh / Hq, h = bh % Hq;
  const int hk = h / (Hq / Hkv);
  const int off = Skv - Sq;
  const int wave_row0 = qtile * BR + qb * 32;
  const int row = wave_row0 + n;
  const bool valid = row < Sq;

  const uint16_t* Kh = K + (int64_t)(b * Hkv + hk) * Skv * D;
  const uint16_t* Vh = V + (int64_t)(b * Hkv + hk) * Skv * D;
  const int last_row = min(qtile * BR + BR, Sq) - 1;
  const int kv_end = CAUSAL ? min(Skv, last_row + off + 1) : Skv;
  const int n_tiles = (kv_end + BC - 1) / BC;
  // Sliding window of `window` keys (causal only, 0 = none): row i sees
  // keys [i + off - window + 1, i + off]; the loop starts at the first tile
  // the workgroup's first row can see.
  const bool win = WIN;   // instantiated for causal calls with window > 0 only
  const int t0 = win ? max(0, qtile * BR + off - window + 1) / BC : 0;

  // K/V tiles through buffer loads; rows past Skv arrive as zeros (masked).
  TileDma<D, BC, NQW> dma;   // the group's tiles, moved by its NQW waves
  dma.init(qb, lane);
  dma.load(Kh, Skv, sK0 + go, (t0 + hg) * BC, qb);
  dma.load(Vh, Skv, sV0 + go, (t0 + hg) * BC, qb);

  const int qrow = min(row, Sq - 1);
  const uint16_t* Qr = Q + ((int64_t)bh * Sq + qrow) * D;
  const uint16_t* dOr = dO + ((int64_t)bh * Sq + qrow) * D;
  u32x4 qreg[NDC], greg[NDC];
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    qreg[c] = *(const u32x4*)(Qr + c * 16 + 8 * g);
    greg[c] = *(const u32x4*)(dOr + c * 16 + 8 * g);
  }
  // D over this lane's half of the columns, plus the other half (lane ^ 32).
  const uint16_t* Or = O + ((int64_t)bh * Sq + qrow) * D;
  float dacc = 0.f;
#pragma unroll
  for (int c = 0; c < NDC; ++c) {
    const u32x4 ov = *(const u32x4*)(Or + c * 16 + 8 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dacc = fmaf(__uint_as_float(ov[i] << 16), __uint_as_float(greg[c][i] << 16), dacc);
      dacc = fmaf(__uint_as_float(ov[i] & 0xffff0000u), __uint_as_float(greg[c][i] & 0xffff0000u),
                  dacc);
    }
  }
  dacc = halfwave_sum(dacc);
  const float dd = valid ? dacc : 0.f;
  // A row with no allowed key (LSE = -inf, possible with a bias) gets
  // probabilities 0, like the padding rows.
  const float lse_row = valid ? LSE[(int64_t)bh * Sq + qrow] : kNegInf;
  const float nl = lse_row != kNegInf ? -lse_row * kLog2e : kNegInf;
  if (g == 0 && hg == 0 && row < Sqp) *(f32x2*)(ws + 2 * ((int64_t)bh * Sqp + row)) = f32x2{dd, nl};
  f32x16 dqt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqt[db][i] = 0.f;

  const int row_limit = CAUSAL ? min(row + off + 1, Skv) : Skv;   // keys [row_lo, row_limit)
  const int row_lo = win ? row + off - window + 1 : 0;
  const float* brow = BIAS ? bias + b * bsb + h * bsh + (int64_t)qrow * Skv : nullptr;
  const int wave_kv_last = CAUSAL ? min(Skv, min(wave_row0 + 31, Sq - 1) + off + 1) - 1 : Skv - 1;
  const int wave_kv_first = win ? wave_row0 + off - window + 1 : 0;
  const int wave_lo_max = win ? min(wave_row0 + 31, Sq - 1) + off - window + 1 : 0;
  int r_off[kRowOffs<D>], t_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, r_off);
  tr_read_offsets<D>(lane, t_off);

  auto step = [&](const uint16_t* cK0, const uint16_t* cV0, uint16_t* nK0, uint16_t* nV0,
                  int tt) {
    const int k0 = tt * BC;
    wait_vmcnt0();   // this wave's part of tile tt has landed
    lds_barrier();   // ... and every wave's; the other buffers are free
    opaque_offsets<kRowOffs<D>>(r_off);
    opaque_offsets<kTrOffs<D>>(t_off);
    if (tt + HS < n_tiles) {
      dma.load(Kh, Skv, nK0 + go, k0 + HS * BC, qb);
      dma.load(Vh, Skv, nV0 + go, k0 + HS * BC, qb);
    }
    if (HS > 1 && tt >= n_tiles) return;   // the group has no tile left (its last step)
    const uint16_t* cK = cK0 + go;
    const uint16_t* cV = cV0 + go;
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      const int ks = k0 + kb * 32;
      if (ks > wave_kv_last || ks + 31 < wave_kv_first) continue;
      const bool need_mask = (ks + 32 > Skv) || (CAUSAL && ks + 31 > wave_row0 + off) ||
                             (win && ks < wave_lo_max);
      // Additive bias of this lane's query for keys ks + 16c + 8g + 0..7
      // (bv[2c], bv[2c + 1]), requested before the products.
      f32x4 bv[4];
      if constexpr (BIAS) {
        if (ks + 32 <= Skv) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bv[e] = *(const f32x4*)(brow + ks + 16 * (e >> 1) + 8 * g + 4 * (e & 1));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int x = 0; x < 4; ++x)
              bv[e][x] = brow[min(ks + 16 * (e >> 1) + 8 * g + 4 * (e & 1) + x, Skv - 1)];
        }
      }
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      const uint16_t* kbp = cK + kb * 32 * D;
      const uint16_t* vbp = cV + kb * 32 * D;
#pragma unroll
      for (int c = 0; c < NDC; ++c) {
        const int o = row_off<D>(r_off, c);
        s = mfma32(lds_row(kbp, o), qreg[c], s);
        dp = mfma32(lds_row(vbp, o), greg[c], dp);
      }
      // dS^T = P^T (dP^T - D); only this step is inside the mask branch.
      u32x4 dsb[2];
      auto softmax = [&](auto masked) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float dsv[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const int i = 8 * c + 2 * j + u;
              const float pre =
                  BIAS ? fmaf(bv[2 * c + (j >> 1)][2 * (j & 1) + u], kLog2e, nl) : nl;
              float p = fast_exp2(fmaf(s[i], scale_log2, pre));
              if constexpr (decltype(masked)::value) {
                const int kk = ks + 16 * c + 8 * g + 2 * j + u;
                p = (kk < row_limit && kk >= row_lo) ? p : 0.f;
              }
              dsv[u] = p * (dp[i] - dd);
            }
            dsb[c][j] = pack_bf16x2(dsv[0], dsv[1]);
          }
      };
      if (need_mask)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dqt[db] = mfma32(tr_col8<D>(kbp + 16 * c * D, t_off, db), dsb[c], dqt[db]);
        }
    }
  };
  if constexpr (HS == 1) {
#pragma clang loop unroll(disable)
    for (int tt = t0; tt < n_tiles; tt += 2) {
      step(sK0, sV0, sK1, sV1, tt);
      if (tt + 1 < n_tiles) step(sK1, sV1, sK0, sV0, tt + 1);
    }
  } else {
    // Every group takes the same number of steps (barriers), the last one
    // possibly without a tile.
    const int n_steps = (max(0, n_tiles - t0) + HS - 1) / HS;
#pragma clang loop unroll(disable)
    for (int i = 0; i < n_steps; i += 2) {
      step(sK0, sV0, sK1, sV1, t0 + hg + HS * i);
      if (i + 1 < n_steps) step(sK1, sV1, sK0, sV0, t0 + hg + HS * (i + 1));
    }
    wait_vmcnt0();   // nothing in flight into LDS
    // Groups 1 .. HS-1 add their dQ sums into group 0's: eight values per
    // lane and round, as 32-byte rows per lane of the wave's region.
    float* red = reinterpret_cast<float*>(sK0);
#pragma unroll
    for (int rd = 0; rd < 2 * NDB; ++rd) {
      lds_barrier();   // the buffers (and the previous round) are no longer read
      f32x16& A = dqt[rd / 2];
      const int e0 = 8 * (rd % 2);
      if (hg > 0) {
        float* dst = red + ((hg - 1) * NQW + qb) * 512 + lane * 8;
        *(f32x4*)dst = f32x4{A[e0], A[e0 + 1], A[e0 + 2], A[e0 + 3]};
        *(f32x4*)(dst + 4) = f32x4{A[e0 + 4], A[e0 + 5], A[e0 + 6], A[e0 + 7]};
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's writes are done
      lds_barrier();
      if (hg == 0) {
#pragma unroll
        for (int hh = 1; hh < HS; ++hh) {
          const float* src = red + ((hh - 1) * NQW + qb) * 512 + lane * 8;
          const f32x4 a = *(const f32x4*)src, c = *(const f32x4*)(src + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            A[e0 + j] += a[j];
            A[e0 + 4 + j] += c[j];
          }
        }
      }
    }
    if (hg > 0) return;
  }
  if (!valid) return;
  store_transposed<NDB>(dQ + ((int64_t)bh * Sq + row) * D, dqt, g, scale);
}

template <int D, bool CAUSAL, bool WIN, bool BIAS>
static hipError_t launch_bwd_w(const BwdArgs& a) {
  const int Sqp = (a.Sq + 31) / 32 * 32;
  const int64_t rows_pad = (int64_t)a.B * a.Hq * Sqp;
  const float sl2 = a.scale * kLog2e;
  // dQ first: it also writes the (D, nl) pairs the dK/dV kernel reads.
  const int BH = a.B * a.Hq;
  auto dq = [&](auto nqw, auto hs) {
    constexpr int NQW = decltype(nqw)::value, HS = decltype(hs)::value;
    const int n_qtiles = (a.Sq + 32 * NQW - 1) / (32 * NQW);
    ATTN_LAUNCH(0, (bwd_dq_kernel<D, CAUSAL, WIN, BIAS, NQW, HS>), dim3(n_qtiles * BH),
                dim3(64 * NQW * HS), a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                (const uint16_t*)a.v, (const uint16_t*)a.d_o, (const uint16_t*)a.o, a.lse, a.ws,
                (uint16_t*)a.dq, BH, a.Hq, a.Hkv, a.Sq, Sqp, a.Skv, a.window, a.bias,
                a.bias_sb, a.bias_sh, a.scale, sl2, n_qtiles);
  };
  {
    using J1 = std::integral_constant<int, 1>;
    using J2 = std::integral_constant<int, 2>;
    using J4 = std::integral_constant<int, 4>;
    if constexpr (D <= 128) {
      int nqw, hs;
      bwd_dq_config(a, &nqw, &hs);
      if (nqw == 2 && hs == 4)
        dq(J2{}, J4{});
      else if (nqw == 4 && hs == 2)
        dq(J4{}, J2{});
      else
        dq(J4{}, J1{});
    } else {
      dq(J4{}, J1{});
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BHk = a.B * a.Hkv;
  // At d = 256 a call without the causal mask runs the causal dK/dV kernel
  // with the diagonal past the last key (i + Skv >= every key j for every
  // query i), which masks nothing: the non-causal instantiation does not
  // fit the registers of that head dimension and spills.
  constexpr bool AS_CAUSAL = CAUSAL || (D >= 256 && !WIN);
  const int diag = CAUSAL ? a.Skv - a.Sq : a.Skv;
  int nkw = 4, hs = 1, hsplit = 1;
  bwd_dkdv_config(a, &nkw, &hs, &hsplit);
  // Head split: float32 partials after the (D, nl) pairs in the workspace.
  float* part = a.ws + bwd_split_part_offset(a.B, a.Hq, a.Sq);
  auto dkdv = [&](auto nkw_c, auto hs_c, auto ps_c) {
    constexpr int NKW = decltype(nkw_c)::value, HS = decltype(hs_c)::value;
    constexpr bool PS = decltype(ps_c)::value;
    const int n_ktiles = (a.Skv + 32 * NKW - 1) / (32 * NKW);
    ATTN_LAUNCH(1, (bwd_dkdv_kernel<D, AS_CAUSAL, WIN, BIAS, false, NKW, HS, PS>),
                dim3(n_ktiles * BHk * (PS ? hsplit : 1)), dim3(64 * NKW * HS), a.stream,
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                (const uint16_t*)a.d_o, (const float*)a.ws, (uint16_t*)a.dk, (uint16_t*)a.dv,
                BHk, a.Hq, a.Hkv, a.Sq, Sqp, a.Skv, a.window, a.bias, a.bias_sb, a.bias_sh,
                a.scale, sl2, rows_pad, diag, nullptr, PS ? hsplit : 1,
                PS ? part : nullptr);
    if constexpr (PS) {
      if (hipPeekAtLastError() != hipSuccess) return;
      const int64_t nkv = (int64_t)BHk * a.Skv * D;
      const int64_t blocks = std::min<int64_t>((2 * nkv / 8 + 255) / 256, 2048);
      ATTN_LAUNCH(2, bwd_dkdv_reduce_kernel<D>, dim3((unsigned)blocks), dim3(256), a.stream,
                  (const float*)part, (uint16_t*)a.dk, (uint16_t*)a.dv, nkv, hsplit);
    }
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using F = std::false_type;
  using T = std::true_type;
  constexpr bool CAN_SPLIT = !WIN && !BIAS;
  if constexpr (D <= 128) {
    if (CAN_SPLIT && hsplit > 1) {
      if constexpr (CAN_SPLIT) {
        if (nkw == 2 && hs == 4)
          dkdv(I2{}, I4{}, T{});
        else if (nkw == 4 && hs == 2)
          dkdv(I4{}, I2{}, T{});
        else
          dkdv(I4{}, I1{}, T{});
      }
    } else if (nkw == 2 && hs == 4) {
      dkdv(I2{}, I4{}, F{});
    } else if (nkw == 4 && hs == 2) {
      dkdv(I4{}, I2{}, F{});
    } else {
      dkdv(I4{}, I1{}, F{});
    }
  } else {
    if constexpr (CAN_SPLIT) {
      if (hsplit > 1) {
        dkdv(I4{}, I1{}, T{});
        return hipGetLastError();
      }
    }
    dkdv(I4{}, I1{}, F{});
  }
  return hipGetLastError();
}

// The sliding window and the additive bias are template parameters: calls
// without them run the kernels with none of their arithmetic.
template <int D, bool CAUSAL, bool WIN>
static hipError_t launch_bwd_b(const BwdArgs& a) {
  if (a.bias) return launch_bwd_w<D, CAUSAL, WIN, true>(a);
  return launch_bwd_w<D, CAUSAL, WIN, false>(a);
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  if constexpr (CAUSAL) {
    if (a.window > 0) return launch_bwd_b<D, true, true>(a);
  }
  return launch_bwd_b<D, CAUSAL, false>(a);
}

}  // namespace attn
