// Split-KV decode: one query token per (batch, query head) against a long
// KV cache (contiguous, or paged through a block table).  The keys are
// partitioned into n_splits sets (contiguous chunks on the vector-unit
// kernel, dealt 32-key tiles on the matrix-core kernel); each set's
// unnormalised online-softmax state (m, l, acc) is computed independently and
// the states are folded with the monoid merge ("Tang, a compiler that derives
// GPU kernels and bounds how fast they can run", Abstract: online softmax as
// a monoid; "Compilers and Kernels", FlashAttention section, the recurrence's
// state and O_i = o_T / l_T), which is associative and commutative, so any
// partition gives the same result up to rounding.  Scoring one token is a
// matrix-vector product, so the split kernels are bound by streaming K and V
// from HBM: they read each key/value row once for all query heads that share
// it, with the next tile's loads in flight while a tile is used.
#include "common.h"
#include "launch.h"

namespace attn {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int PER16 = 4;  // elements per 16-byte access
  __device__ static void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(x[i]);
  }
  __device__ static void store2(float* p, float a, float b) { *(f32x2*)p = f32x2{a, b}; }
};
template <>
struct Elem<uint16_t> {
  static constexpr int PER16 = 8;
  __device__ static void unpack(u32x4 x, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(x[i] << 16);
      f[2 * i + 1] = __uint_as_float(x[i] & 0xffff0000u);
    }
  }
  __device__ static void store2(uint16_t* p, float a, float b) { *(uint32_t*)p = pack_bf16x2(a, b); }
};

constexpr int kDecodeThreads = 256;

// Persistent split kernel.  A work item is one key chunk (split) of one
// key/value head for up to GC of its query heads.  Each workgroup walks the
// items blockIdx.x, blockIdx.x + gridDim.x, ...; every item is cut into
// stages of SK keys (64 KB of K and V), and the stages of all its items form
// one stream: stage j+1 moves HBM -> LDS (global_load_lds) while stage j is
// scored and accumulated from LDS.  Within an item the per-head state
// (m, l, acc) is merged across stages by the online rescale; at the item's
// end the partial accumulators of the key rows are reduced (lane swaps, then
// LDS across waves) and the item's state is written to the workspace.
template <typename T, int D>
struct DecodeCfg {
  static constexpr int E = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  static constexpr int CPR = D / E;                   // chunks per key row
  static constexpr int LPR = CPR;                     // lanes per key row
  static constexpr int KPP = kDecodeThreads / LPR;    // key rows per pass
  static constexpr int SK = 32768 / (D * (int)sizeof(T));  // keys per stage
  static constexpr int NP = SK / KPP;                 // passes per stage
  static constexpr int STAGE = SK * D;                // elements per tensor per stage
  static constexpr int BLOCKS = STAGE * (int)sizeof(T) / 1024;  // 1 KB DMA blocks per tensor
};

template <typename T, int D>
__device__ __forceinline__ void decode_dma(const T* src, T* dst, int L, int wave, int lane) {
  using C = DecodeCfg<T, D>;
  static_assert(C::BLOCKS % 4 == 0, "stage must split evenly over the waves");
#pragma unroll
  for (int j = 0; j < C::BLOCKS / 4; ++j) {
    const int blk = j * 4 + wave;
    const int pos = blk * 64 + lane;                  // chunk index within the stage
    const int r = min(pos / C::CPR, L - 1);           // rows past the chunk end repeat
    // The cache is read once per step: non-temporal loads.
    __builtin_amdgcn_global_load_lds((const void*)(src + (int64_t)r * D + (pos % C::CPR) * C::E),
                                     (__attribute__((address_space(3))) void*)(dst + blk * 1024 / (int)sizeof(T)),
                                     16, 0, kCacheStream);
  }
}

template <typename T, int D, int GC>
__global__ __launch_bounds__(kDecodeThreads, 1) void decode_split_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    float* __restrict__ ws, int B, int Hq, int Hkv, int Skv, int chunk, int n_splits,
    int n_hchunks, float scale_log2) {
  using C = DecodeCfg<T, D>;
  constexpr int E = C::E, LPR = C::LPR, KPP = C::KPP, SK = C::SK, NP = C::NP;
  constexpr int NW = kDecodeThreads / 64;
  constexpr int RPW = 64 / LPR;  // key rows per wave
  __shared__ __attribute__((aligned(1024))) T sK[2][C::STAGE];
  __shared__ __attribute__((aligned(1024))) T sV[2][C::STAGE];
  __shared__ float sMax[NW][GC];
  __shared__ float sRed[NW][GC][D + 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = wave_id();
  const int sub = tid % LPR;   // chunk (column slice) of this lane
  const int kr = tid / LPR;    // key row within a pass
  const int G = Hq / Hkv;
  const int64_t BHq = (int64_t)B * Hq;
  const int n_items = n_splits * Hkv * n_hchunks * B;
  float* ws_m = ws;
  float* ws_l = ws + (int64_t)n_splits * BHq;
  float* ws_acc = ws + 2 * (int64_t)n_splits * BHq;

  struct Item {
    int split, hk, hc, b, k_begin, L, n_st;
  };
  auto item_of = [&](int it) {
    Item x;
    x.split = it % n_splits;
    int r = it / n_splits;
    x.hc = r % n_hchunks;
    r /= n_hchunks;
    x.hk = r % Hkv;
    x.b = r / Hkv;
    x.k_begin = min(x.split * chunk, Skv);
    x.L = min(x.k_begin + chunk, Skv) - x.k_begin;
    x.n_st = (x.L + SK - 1) / SK;
    return x;
  };
  // Issue the DMA of stage `st` of item `x` into buffer `buf`.
  auto issue = [&](const Item& x, int st, int buf) {
    const int64_t base = ((int64_t)(x.b * Hkv + x.hk) * Skv + x.k_begin + st * SK) * D;
    const int Ls = min(SK, x.L - st * SK);
    decode_dma<T, D>(K + base, sK[buf], Ls, wave, lane);
    decode_dma<T, D>(V + base, sV[buf], Ls, wave, lane);
  };

  int it = blockIdx.x;
  // Skip leading empty items (identity states are written without a stage).
  auto write_identity = [&](const Item& x) {
    const int h0 = x.hk * G + x.hc * GC;
    const int nh = min(GC, G - x.hc * GC);
    for (int i = tid; i < nh * D; i += kDecodeThreads) {
      const int hh = i / D, dd = i % D;
      const int64_t idx = (int64_t)x.split * BHq + (int64_t)x.b * Hq + h0 + hh;
      ws_acc[idx * D + dd] = 0.f;
      if (dd == 0) {
        ws_m[idx] = kNegInf;
        ws_l[idx] = 0.f;
      }
    }
  };
  while (it < n_items && item_of(it).L <= 0) {
    write_identity(item_of(it));
    it += gridDim.x;
  }
  if (it >= n_items) return;

  Item cur = item_of(it);
  int st = 0, buf = 0;
  issue(cur, 0, 0);

  float q[GC][E], m[GC], acc[GC][E];
  KahanSum lsum[GC];
  bool fresh = true;  // first stage of the current item

  while (true) {
    // Next stage in the stream (same item or the next non-empty one).
    Item nxt = cur;
    int nst = st + 1;
    int nit = it;
    if (nst >= cur.n_st) {
      nst = 0;
      nit = it + gridDim.x;
      while (nit < n_items && item_of(nit).L <= 0) {
        write_identity(item_of(nit));
        nit += gridDim.x;
      }
      if (nit < n_items) nxt = item_of(nit);
    }
    const bool has_next = nit < n_items;

    const int h0 = cur.hk * G + cur.hc * GC;
    const int nh = min(GC, G - cur.hc * GC);
    if (fresh) {
#pragma unroll
      for (int hh = 0; hh < GC; ++hh) {
        const int hq = h0 + min(hh, nh - 1);
        float f[E];
        Elem<T>::unpack(*(const u32x4*)(Q + ((int64_t)cur.b * Hq + hq) * D + sub * E), f);
#pragma unroll
        for (int e = 0; e < E; ++e) q[hh][e] = f[e] * scale_log2;
        m[hh] = kNegInf;
        lsum[hh] = KahanSum{0.f, 0.f};
#pragma unroll
        for (int e = 0; e < E; ++e) acc[hh][e] = 0.f;
      }
      fresh = false;
    }

    wait_vmcnt0();     // this wave's part of the current stage is in LDS
    __syncthreads();   // every wave's part; the other buffer is free
    if (has_next) issue(nxt, nst, buf ^ 1);

    const T* cK = sK[buf];
    const T* cV = sV[buf];
    const int Ls = min(SK, cur.L - st * SK);
    float s[GC][NP], tmax[GC];
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) tmax[hh] = kNegInf;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = p * KPP + kr;
      float f[E];
      Elem<T>::unpack(*(const u32x4*)(cK + r * D + sub * E), f);
#pragma unroll
      for (int hh = 0; hh < GC; ++hh) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaf(q[hh][e], f[e], a);
        a = group_reduce<LPR, false>(a);
        s[hh][p] = (r < Ls) ? a : kNegInf;
        tmax[hh] = fmaxf(tmax[hh], s[hh][p]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {
      float x = tmax[hh];
      if constexpr (LPR < 16) x = group_reduce<16, true>(x);
      if constexpr (LPR < 32) {
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      if constexpr (LPR < 64) x = halfwave_max(x);
      if (lane == 0) sMax[wave][hh] = x;
    }
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {
      float mx = sMax[0][hh];
#pragma unroll
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, sMax[w][hh]);
      const float mnew = fmaxf(m[hh], mx);           // finite: the stage is non-empty
      const float alpha = fast_exp2(m[hh] - mnew);   // 0 on the item's first stage
      m[hh] = mnew;
      lsum[hh].scale(alpha);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hh][e] *= alpha;
    }
    // The stage's terms are summed from zero and then added to the running
    // (lsum, acc): added one by one, terms far below a large running value
    // (keys after a dominant one, over millions of keys) would round away.
    float lst[GC], ast[GC][E];
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {
      lst[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) ast[hh][e] = 0.f;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int r = p * KPP + kr;
      float f[E];
      Elem<T>::unpack(*(const u32x4*)(cV + r * D + sub * E), f);
#pragma unroll
      for (int hh = 0; hh < GC; ++hh) {
        const float pw = fast_exp2(s[hh][p] - m[hh]);
        lst[hh] += pw;
#pragma unroll
        for (int e = 0; e < E; ++e) ast[hh][e] = fmaf(pw, f[e], ast[hh][e]);
      }
    }
#pragma unroll
    for (int hh = 0; hh < GC; ++hh) {
      lsum[hh].add(lst[hh]);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[hh][e] += ast[hh][e];
    }

    if (st + 1 >= cur.n_st) {
      // Item done: reduce over key rows (rows of a wave by lane swaps, the
      // waves through LDS) and write its state.
#pragma unroll
      for (int hh = 0; hh < GC; ++hh) {
        float l = lsum[hh].value();  // identical across the lanes of a row group
#pragma unroll
        for (int e = 0; e < E; ++e) {
          float x = acc[hh][e];
          if constexpr (RPW >= 2) {
            if constexpr (LPR == 32) {
              auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
              x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            } else if constexpr (LPR == 16) {
              auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
              x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
              x = halfwave_sum(x);
            } else {  // LPR == 8: lanes i and i ^ 8 hold the same columns
              x += dpp_mov<kRowRor8>(x);
              auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
              x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
              x = halfwave_sum(x);
            }
          }
          if (lane < LPR) sRed[wave][hh][sub * E + e] = x;
        }
        if constexpr (RPW >= 2) {
          if constexpr (LPR == 32) {
            l = halfwave_sum(l);
          } else if constexpr (LPR == 16) {
            auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
            l = halfwave_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
          } else {
            l += dpp_mov<kRowRor8>(l);
            auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(l), __float_as_uint(l), false, false);
            l = halfwave_sum(__uint_as_float(r[0]) + __uint_as_float(r[1]));
          }
        }
        if (lane == 0) sRed[wave][hh][D] = l;
      }
      __syncthreads();
      for (int i = tid; i < nh * (D + 1); i += kDecodeThreads) {
        const int hh = i / (D + 1), dd = i % (D + 1);
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += sRed[w][hh][dd];
        const int64_t idx = (int64_t)cur.split * BHq + (int64_t)cur.b * Hq + h0 + hh;
        if (dd < D) {
          ws_acc[idx * D + dd] = t;
        } else {
          ws_l[idx] = t;
          ws_m[idx] = m[hh];
        }
      }
      fresh = true;
    }
    if (!has_next) break;
    // sMax / sRed are rewritten by the next stage only after its barrier.
    cur = nxt;
    st = nst;
    it = nit;
    buf ^= 1;
  }
}

// ---------------------------------------------------------------------------
// bf16 split kernel on the matrix cores.  A work unit is one split (every
// n_splits-th 32-key tile) of one key/value head for up to 8 of its query
// heads.  The query
// heads take the place of the query rows of the forward kernel (32 MFMA
// columns; the ones past the group's heads are fed zeros): per tile of 32
// keys, S^T = K Q^T (lane = head, 16 scores per lane), the running
// (m, l, o) per head, and O^T += V^T P^T with V^T from transpose reads.
//
// Work is assigned per wave: wave w of the grid takes units w, w + W, ...
// (W = waves in the grid).  Each wave streams its units' tiles through its
// own pair of LDS buffers with global_load_lds, tile t+1 in flight while
// tile t is used (across unit boundaries too), and writes each unit's state
// straight from registers.  No barriers: the waves of a workgroup share only
// the LDS allocation.
// ---------------------------------------------------------------------------
constexpr float kDecodeLazy = 8.f;  // lazy rescale threshold (log2 units), as in the forward
constexpr int kDecodeHC = 8;        // query heads per work unit on the matrix cores

template <int D, bool PAGED>
__global__ __launch_bounds__(256, 1) void decode_split_mfma_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ ws, int B, int Hq, int Hkv, int Skv,
    int n_splits, int n_hchunks, float scale_log2, PagedKV pg) {
  constexpr int NDC = D / 16;
  constexpr int NDB = D / 32;
  constexpr int TK = 32;  // keys per tile
  constexpr int HC = kDecodeHC;
  // Each wave's two tile buffers live in separate variables so that the
  // compiler sees the DMA into one cannot alias the reads of the other.
  __shared__ __attribute__((aligned(1024))) uint16_t sKa[4][TK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sKb[4][TK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sVa[4][TK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sVb[4][TK * D];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int n = lane & 31, g = lane >> 5;
  const int G = Hq / Hkv;
  const int64_t BHq = (int64_t)B * Hq;
  const int n_units = n_splits * Hkv * n_hchunks * B;
  const int W = gridDim.x * 4;
  float* ws_m = ws;
  float* ws_l = ws + (int64_t)n_splits * BHq;
  float* ws_acc = ws + 2 * (int64_t)n_splits * BHq;

  // A split takes every n_splits-th 32-key tile of the head's keys (tiles
  // split, split + n_splits, ...): the waves working on the splits of one
  // head then stream one contiguous window of K and V together, which the
  // memory system serves faster than as many separate streams.  Any
  // partition of the keys gives the same merged result.
  //
  // Paged caches: K and V are pools [n_pages, Hkv, page_size, d]; key t of
  // stream b is row t % page_size of page table[b][t / page_size] (a page
  // holds whole 32-key tiles), and stream b has lens[b] keys, clamped to
  // the table's capacity.  A page id outside the pool reads as zeros.
  struct Unit {
    int split, hk, hc, b;
    int keys;   // keys of the unit's stream
    int L;      // tiles of this split
  };
  auto unit_of = [&](int u) {
    Unit x;
    x.split = u % n_splits;
    int r = u / n_splits;
    x.hc = r % n_hchunks;
    r /= n_hchunks;
    x.hk = r % Hkv;
    x.b = r / Hkv;
    x.keys = PAGED ? min(max(pg.lens[x.b], 0), pg.max_pages * pg.page_size) : Skv;
    const int tiles = (x.keys + TK - 1) / TK;
    x.L = x.split < tiles ? (tiles - x.split + n_splits - 1) / n_splits : 0;
    return x;
  };
  auto n_tiles = [&](const Unit& x) { return x.L; };
  auto tile_of = [&](const Unit& x, int t) { return x.split + t * n_splits; };
  TileDma<D, TK, 1> pdma;   // paged tiles: one buffer descriptor per page
  if constexpr (PAGED) pdma.init(0, lane);
  // Page id of tile t of unit x, as a vector load (the address is made
  // opaque per lane) so that the wait for it is the wait for the tiles in
  // flight, issued one step before the id is needed.
  auto load_pid = [&](const Unit& x, int t) -> int {
    int z = lane;
    asm volatile("" : "+v"(z));
    const int page = tile_of(x, t) * TK / pg.page_size;   // < max_pages
    return pg.table[(int64_t)x.b * pg.max_pages + page + (z >> 30)];
  };
  auto issue = [&](const Unit& x, int t, int pid, uint16_t* dK, uint16_t* dV) {
    if constexpr (PAGED) {
      const int p = __builtin_amdgcn_readfirstlane(pid);
      const bool ok = p >= 0 && p < pg.n_pages;
      const int64_t base = ((int64_t)(ok ? p : 0) * Hkv + x.hk) * pg.page_size * D;
      const int r0 = tile_of(x, t) * TK % pg.page_size;
      // The cache is read once per step: non-temporal loads.
      pdma.template load<kCacheStream>(K + base, ok ? pg.page_size : 0, dK, r0, 0);
      pdma.template load<kCacheStream>(V + base, ok ? pg.page_size : 0, dV, r0, 0);
    } else {
      const int64_t base = (int64_t)(x.b * Hkv + x.hk) * Skv * D;
      const int r0 = tile_of(x, t) * TK;
      dma_tile<D, TK, 1, kCacheStream>(K + base, dK, r0, Skv, 0, lane);
      dma_tile<D, TK, 1, kCacheStream>(V + base, dV, r0, Skv, 0, lane);
    }
  };
  // Raw query rows of the unit's heads (lanes past the group's heads load a
  // valid row and are zeroed by q_keep when the rows are adopted, so that
  // no instruction depends on the load before the unit starts).
  auto load_q = [&](const Unit& x, u32x4* qr) {
    const int nh = min(HC, G - x.hc * HC);
    const int hq = x.hk * G + x.hc * HC + min(n, nh - 1);
    const uint16_t* qp = Q + ((int64_t)x.b * Hq + hq) * D + 8 * g;
#pragma unroll
    for (int c = 0; c < NDC; ++c) qr[c] = *(const u32x4*)(qp + c * 16);
  };
  // A zero scale makes every score 0: the query rows are replaced by zeros
  // and the scale by 1 (the same exact scores; keys past the end stay -inf,
  // where -inf times a zero scale would be NaN).
  const bool zero_scale = scale_log2 == 0.f;
  auto q_keep = [&](const Unit& x) {
    return (n < min(HC, G - x.hc * HC) && !zero_scale) ? 0xffffffffu : 0u;
  };
  auto write_state = [&](const Unit& x, float m, float lpart, const f32x16* oacc) {
    const int nh = min(HC, G - x.hc * HC);
    const float l = halfwave_sum(lpart);
    if (n < nh) {
      const int64_t idx =
          (int64_t)x.split * BHq + (int64_t)x.b * Hq + x.hk * G + x.hc * HC + n;
      float* dst = ws_acc + idx * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *(f32x4*)(dst + db * 32 + 8 * i4 + 4 * g) =
              f32x4{oacc[db][4 * i4], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2], oacc[db][4 * i4 + 3]};
      if (g == 0) {
        ws_m[idx] = m;   // log2 domain, like every partial
        ws_l[idx] = l;
      }
    }
  };

  int u = blockIdx.x * 4 + wave;
  // Units with no keys get the identity state and no tiles.
  while (u < n_units && unit_of(u).L <= 0) {
    f32x16 z[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) z[db][i] = 0.f;
    write_state(unit_of(u), kNegInf, 0.f, z);
    u += W;
  }
  if (u >= n_units) return;

  const uint32_t qsign = scale_log2 < 0.f ? 0x80008000u : 0u;
  const float c2 = zero_scale ? 1.f : fabsf(scale_log2);
  int r_off[kRowOffs<D>], t_off[kTrOffs<D>];
  row_read_offsets<D>(n, g, r_off);
  tr_read_offsets<D>(lane, t_off);

  Unit cur = unit_of(u);
  u32x4 qreg[NDC], qnext[NDC];
  load_q(cur, qreg);
  {
    const uint32_t keep = q_keep(cur);
#pragma unroll
    for (int c = 0; c < NDC; ++c) qreg[c] &= keep;
  }
  issue(cur, 0, PAGED ? load_pid(cur, 0) : 0, sKa[wave], sVa[wave]);
  int t = 0;
  bool new_q = false;
  float m_ref = kNegInf;
  KahanSum lpart{0.f, 0.f};
  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  // One tile of this wave's stream; returns false after the last tile.
  auto step = [&](const uint16_t* cK, const uint16_t* cV, uint16_t* nK, uint16_t* nV) -> bool {
    const int nt = n_tiles(cur);
    Unit nxt = cur;
    int tn = t + 1, un = u;
    const bool unit_end = tn >= nt;
    if (unit_end) {
      tn = 0;
      un = u + W;
      while (un < n_units && unit_of(un).L <= 0) {
        f32x16 z[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) z[db][i] = 0.f;
        write_state(unit_of(un), kNegInf, 0.f, z);
        un += W;
      }
      if (un < n_units) nxt = unit_of(un);
    }
    const bool more = un < n_units;
    const bool go_on = !unit_end || more;
    int pid = 0;
    if (PAGED && go_on) pid = load_pid(nxt, tn);

    wait_vmcnt0();   // tile t (and every earlier load of this wave) has landed
    if (new_q) {
      const uint32_t keep = q_keep(cur);
#pragma unroll
      for (int c = 0; c < NDC; ++c) qreg[c] = qnext[c] & keep;
      new_q = false;
    }
    if (go_on) {
      issue(nxt, tn, pid, nK, nV);
      if (unit_end) load_q(nxt, qnext);
    }

    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int c = 0; c < NDC; ++c)
      s = mfma32(lds_row(cK, row_off<D>(r_off, c)), qreg[c] ^ qsign, s);
    const int kvalid = cur.keys - tile_of(cur, t) * TK;  // keys of this tile that exist
    float rmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = 16 * (i >> 3) + 8 * g + (i & 7);
      s[i] = (kk < kvalid) ? s[i] : kNegInf;
      rmax = fmaxf(rmax, s[i]);
    }
    const float mnew = fmaxf(m_ref, halfwave_max(rmax) * c2);
    if (__any(mnew > m_ref + kDecodeLazy)) {
      const float alpha = (mnew == kNegInf) ? 1.f : fast_exp2(m_ref - mnew);
      lpart.scale(alpha);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      m_ref = mnew;
    }
    const float msub = (m_ref == kNegInf) ? 0.f : m_ref;
    u32x4 pb[2];
    float tl = 0.f;   // the tile's sum, added to lpart as one term
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float p0 = fast_exp2(fmaf(s[8 * c + 2 * j], c2, -msub));
        const float p1 = fast_exp2(fmaf(s[8 * c + 2 * j + 1], c2, -msub));
        tl += p0 + p1;
        pb[c][j] = pack_bf16x2(p0, p1);
      }
    lpart.add(tl);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = mfma32(tr_col8<D>(cV + 16 * c * D, t_off, db), pb[c],
                          oacc[db]);

    if (unit_end) {
      write_state(cur, m_ref, lpart.value(), oacc);
      if (!more) return false;
      m_ref = kNegInf;
      lpart = KahanSum{0.f, 0.f};
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
      new_q = true;
      cur = nxt;
      u = un;
    }
    t = tn;
    return true;
  };
  while (step(sKa[wave], sVa[wave], sKb[wave], sVb[wave]) &&
         step(sKb[wave], sVb[wave], sKa[wave], sVa[wave])) {
  }
}

// One wave per query (b, h): lanes hold the split states (m_s, l_s) in
// parallel, the wave computes M = max_s m_s and the weights exp2(m_s - M)
// (identity states, m_s = -inf, weigh 0), then every lane folds two output
// columns over the splits: O = sum_s w_s acc_s / sum_s w_s l_s and
// LSE = (M + log2 l) ln 2.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ ws,
                                                             T* __restrict__ O,
                                                             float* __restrict__ LSE, int BHq,
                                                             int n_splits) {
  constexpr int CPL = D / 64;  // columns per lane (1, 2 or 4)
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= BHq) return;
  const float* ws_m = ws;
  const float* ws_l = ws + (int64_t)n_splits * BHq;
  const float* ws_acc = ws + 2 * (int64_t)n_splits * BHq;
  T* o = O + (int64_t)bh * D + lane * CPL;
  if (n_splits <= 16) {
    // Up to 16 splits: every load of the query head is issued before any
    // result is used (one memory round trip).  Lane s < n_splits holds
    // (m_s, l_s); each lane holds its columns of all the accumulators.
    const int sl = min(lane, n_splits - 1);
    const float ms = ws_m[(int64_t)sl * BHq + bh];
    const float ls = ws_l[(int64_t)sl * BHq + bh];
    float v[16][CPL];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float* src = ws_acc + ((int64_t)min(j, n_splits - 1) * BHq + bh) * D + lane * CPL;
#pragma unroll
      for (int c = 0; c < CPL; ++c) v[j][c] = src[c];
    }
    const bool own = lane < n_splits;
    const float M = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(
                   __builtin_bit_cast(int, group_reduce<16, true>(own ? ms : kNegInf))));
    const float w = (own && ms != kNegInf) ? fast_exp2(ms - M) : 0.f;
    const float l = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(
                   __builtin_bit_cast(int, group_reduce<16, false>(w * ls))));
    float a[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) a[c] = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float wj =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
#pragma unroll
      for (int c = 0; c < CPL; ++c) a[c] = fmaf(wj, v[j][c], a[c]);
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;   // a stream with no keys: O = 0
    if constexpr (CPL == 1) {
      if constexpr (sizeof(T) == 4) {
        o[0] = a[0] * inv;
      } else {
        o[0] = f32_to_bf16(a[0] * inv);
      }
    } else {
#pragma unroll
      for (int c = 0; c < CPL; c += 2) Elem<T>::store2(o + c, a[c] * inv, a[c + 1] * inv);
    }
    if (LSE && lane == 0) LSE[bh] = (M + fast_log2(l)) * kLn2;
    return;
  }
  float M = kNegInf;
  for (int s = lane; s < n_splits; s += 64) M = fmaxf(M, ws_m[(int64_t)s * BHq + bh]);
  M = group_reduce<64, true>(M);
  float l = 0.f, a[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) a[c] = 0.f;
  for (int s0 = 0; s0 < n_splits; s0 += 64) {
    const int s = s0 + lane;
    float w = 0.f;
    if (s < n_splits) {
      const float ms = ws_m[(int64_t)s * BHq + bh];
      w = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
      l = fmaf(w, ws_l[(int64_t)s * BHq + bh], l);
    }
    const int ns = min(64, n_splits - s0);
    // Groups of 16 splits: all loads of a group are issued before use.
    for (int j0 = 0; j0 < ns; j0 += 16) {
      float v[16][CPL];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int sj = s0 + min(j0 + j, ns - 1);
        const float* src = ws_acc + ((int64_t)sj * BHq + bh) * D + lane * CPL;
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[j][c] = src[c];
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float wj = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(j0 + j, 63)));
        const float wjm = (j0 + j < ns) ? wj : 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) a[c] = fmaf(wjm, v[j][c], a[c]);
      }
    }
  }
  l = group_reduce<64, false>(l);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if constexpr (CPL == 1) {
    if constexpr (sizeof(T) == 4) {
      o[0] = a[0] * inv;
    } else {
      o[0] = f32_to_bf16(a[0] * inv);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CPL; c += 2) Elem<T>::store2(o + c, a[c] * inv, a[c + 1] * inv);
  }
  if (LSE && lane == 0) LSE[bh] = (M + fast_log2(l)) * kLn2;
}

template <typename T, int D, int GC>
static hipError_t launch_decode_t(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  const int n_hchunks = (G + GC - 1) / GC;
  const int chunk = (a.Skv + a.n_splits - 1) / a.n_splits;
  const int n_items = a.n_splits * a.Hkv * n_hchunks * a.B;
  const int grid = n_items < device_cus() ? n_items : device_cus();
  ATTN_LAUNCH(0, (decode_split_kernel<T, D, GC>), dim3(grid), dim3(kDecodeThreads),
              a.stream, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.ws, a.B, a.Hq,
              a.Hkv, a.Skv, chunk, a.n_splits, n_hchunks, a.scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BHq = a.B * a.Hq;
  ATTN_LAUNCH(1, (decode_combine_kernel<T, D>), dim3((BHq + 3) / 4), dim3(256), a.stream,
              (const float*)a.ws, (T*)a.o, a.lse, BHq, a.n_splits);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t dispatch_decode_g(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  if (G == 1) return launch_decode_t<T, D, 1>(a);
  if (G == 2) return launch_decode_t<T, D, 2>(a);
  if constexpr (D > 128) {
    return launch_decode_t<T, D, 4>(a);  // 8 heads x 256 columns exceed the LDS budget
  } else {
    if (G <= 4) return launch_decode_t<T, D, 4>(a);
    return launch_decode_t<T, D, 8>(a);
  }
}

template <int D>
static hipError_t launch_decode_mfma(const DecodeArgs& a) {
  const int G = a.Hq / a.Hkv;
  const int n_hchunks = (G + kDecodeHC - 1) / kDecodeHC;
  const int n_units = a.n_splits * a.Hkv * n_hchunks * a.B;
  // One workgroup (four waves) per compute unit, each wave a stream of units.
  const int wgs = (n_units + 3) / 4;
  const int grid = wgs < device_cus() ? wgs : device_cus();
  if (a.pg.table)
    ATTN_LAUNCH(0, (decode_split_mfma_kernel<D, true>), dim3(grid), dim3(256), a.stream,
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ws,
                a.B, a.Hq, a.Hkv, 0, a.n_splits, n_hchunks, a.scale * kLog2e, a.pg);
  else
    ATTN_LAUNCH(0, (decode_split_mfma_kernel<D, false>), dim3(grid), dim3(256), a.stream,
                (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.ws,
                a.B, a.Hq, a.Hkv, a.Skv, a.n_splits, n_hchunks, a.scale * kLog2e,
                PagedKV{nullptr, nullptr, 0, 0, 0});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int BHq = a.B * a.Hq;
  ATTN_LAUNCH(1, (decode_combine_kernel<uint16_t, D>), dim3((BHq + 3) / 4), dim3(256),
              a.stream, (const float*)a.ws, (uint16_t*)a.o, a.lse, BHq, a.n_splits);
  return hipGetLastError();
}

template <typename T>
static hipError_t dispatch_decode_d(const DecodeArgs& a) {
  if constexpr (sizeof(T) == 2) {
    if (a.d == 64) return launch_decode_mfma<64>(a);
    if (a.d == 128) return launch_decode_mfma<128>(a);
  }
  if (a.pg.table) return hipErrorInvalidValue;   // paged caches: bf16, d 64 / 128 only
  switch (a.d) {
    case 64: return dispatch_decode_g<T, 64>(a);
    case 128: return dispatch_decode_g<T, 128>(a);
    case 256: return dispatch_decode_g<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.dtype == 0 ? dispatch_decode_d<float>(a) : dispatch_decode_d<uint16_t>(a);
}

}  // namespace attn
