// Tile and launch selection for the bf16 forward: a per-tile time estimate
// picks the waves per workgroup (NW, 32 query rows each) and keys per tile
// (BC) among the compiled candidates, per call shape.
//
// "Tang, a compiler that derives GPU kernels and bounds how fast they can
// run", Abstract: a per-tile traffic and time estimate chooses the tile; and
// "Compilers and Kernels", section "Tiling maps work onto finite resources":
// a tile choice holds for a shape, dtype and device, so the cached choice is
// keyed by every fact it depends on (head dim, causal, B, Hq, Hkv, Sq, Skv,
// the device's compute units and the candidate's occupancy there).
//
// The estimate, for candidate (NW, BC) at head dim D, in SIMD cycles:
//  * a wave computing a key tile costs  M + V + L - O  and waiting on one
//    F = Fill + kSyncPerTile:
//      M = BC D / 8       matrix-core cycles: BC/32 * D/16 QK^T products and
//                         as many PV products, 32 cycles each;
//      V = kValuPer32 BC/32   softmax on the vector unit (per lane BC/2
//                         scores: an FMA, an exp2 at quarter rate, an add,
//                         half a conversion);
//      L = 4 BC D / kLdsPerSimd   the K rows and transposed V rows it reads
//                         from LDS;
//      O = kOverlap2 or kOverlap3 (per 32 keys) with two, or three or more,
//                         waves per SIMD: what the other waves' products hide
//                         of a wave's vector and LDS work;
//      Fill = kFillPerD D / NW * BC/32   the wave's share of moving the K/V
//                         tile into LDS (fewer waves, larger share);
//  * a wave waits on every tile of its workgroup but computes only those
//    up to its own last row (causal); a workgroup takes as long as its
//    busiest SIMD (one wave per SIMD, two for NW = 8);
//  * plus a per-workgroup prologue (a transfer latency, then its Q rows and
//    first K/V tile at one compute unit's share of the HBM bandwidth, since
//    every unit starts a workgroup at once) and epilogue (O and LSE stores),
//    hidden by the other workgroups resident on its compute unit;
//  * workgroups are dealt in launch order (heaviest query tile first when
//    causal) to the earliest-free of max(1, 4 / NW) "machines" per compute
//    unit; the estimate is the makespan plus a launch latency, at 2.4 GHz.
// The waves per SIMD come from the runtime's occupancy for the compiled
// kernel (registers, LDS) and from the grid when it is smaller.  The
// constants were calibrated once on MI355X against timed sweeps of all
// candidates on twelve shapes (the bench's calibration shapes); the bench
// times all candidates on those and on eight more shapes that took no part
// in the calibration, and reports each pick against the fastest.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <queue>
#include <unordered_map>
#include <vector>

#include "launch.h"

namespace attn {

hipError_t fwd_candidate_fn(int d, bool causal, int idx, const void** fn);

namespace {

// nw waves per workgroup in `split` key groups of nw / split waves; group
// g takes the bc-key tiles g, g + split, ...; 32 nw / split query rows per
// workgroup.  split = nw is the key-split kernel (one 32-row block).
struct Cand {
  int nw, bc, split;
};

// Candidates per head dim, in the order of fwd_candidate_i in fwd.hip.
const Cand kCand64[] = {{4, 64, 1}, {4, 32, 1}, {8, 64, 1}, {2, 64, 1},
                        {4, 32, 4}, {2, 32, 2}, {4, 64, 2}};
const Cand kCand128[] = {{4, 32, 1}, {4, 64, 1}, {8, 32, 1}, {8, 64, 1},
                         {4, 32, 4}, {2, 32, 2}, {4, 32, 2}};
const Cand kCand256[] = {{8, 32, 1}, {4, 32, 1}};

int candidates(int d, const Cand** out) {
  switch (d) {
    case 64: *out = kCand64; return 7;
    case 128: *out = kCand128; return 7;
    case 256: *out = kCand256; return 2;
  }
  *out = nullptr;
  return 0;
}

constexpr double kClockGHz = 2.4;
constexpr double kValuPer32 = 400.0;     // softmax cycles per 32 keys and wave
constexpr double kLdsPerSimd = 45.0;     // LDS bytes per cycle one SIMD's waves read
constexpr double kOverlap2 = 300.0;      // hidden per 32 keys at 2 waves per SIMD
constexpr double kOverlap3 = 500.0;      // ... at 3 or more
constexpr double kFillPerD = 12.0;       // K/V tile fill cycles per head-dim column
constexpr double kSyncPerTile = 250.0;   // barrier round per tile
constexpr double kPrologue = 4800.0;     // first-transfer latency of a workgroup
constexpr double kPrologueBytesPerCycle = 10.0;   // its Q rows and first K/V tile, at a
                                                 // compute unit's share of HBM
constexpr double kEpilogue = 400.0;      // O and LSE stores
constexpr double kLaunchUs = 4.0;        // launch and first-wave latency
constexpr double kKsFillPerD = 16.0;     // key split: a wave's own K/V tile per column
constexpr double kKsPrologue = 2400.0;   // key split: first-transfer latency
constexpr double kKsMerge = 3000.0;      // key split: the states' merge through LDS
constexpr double kSplitMerge = 1500.0;   // two key groups: the second's state merged into the first

// Workgroups per compute unit of candidate (d, causal, idx), from the
// runtime's occupancy calculator (registers and LDS of the compiled kernel).
int occupancy(int d, bool causal, int idx, int nw) {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int key = ((dev * 512 + d) * 2 + (causal ? 1 : 0)) * 8 + idx;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  const void* fn = nullptr;
  int n = 0;
  if (fwd_candidate_fn(d, causal, idx, &fn) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, 64 * nw, 0) != hipSuccess || n <= 0)
    n = 1;
  cache[key] = n;
  return n;
}

struct Shape {
  int d, causal, B, Hq, Hkv, Sq, Skv;
};

// Key-split candidate (|nw| waves on one 32-row query block, each with its
// own tiles and state, merged at the end).  A wave moves its whole tile
// (kKsFillPerD D cycles, no sharing), reads only V from LDS and has no
// barrier; its workgroup takes as long as its busiest wave, ceil(n_t / NW)
// tiles, plus the merge.  Every K/V tile is fetched once per wave instead of
// once per workgroup, so the candidate only runs where the plain kernels
// leave compute units idle: at most one 32-row query block per compute unit.
double estimate_ks_us(const Shape& s, int NW, int occ, int cus) {
  const int D = s.d, BC = 32;
  const int off = s.Skv - s.Sq;
  const int n_qt = (s.Sq + 31) / 32;
  const int64_t n_wg = (int64_t)n_qt * s.B * s.Hq;
  if (n_wg > cus) return INFINITY;
  const double per_cu = std::min<double>(occ, (double)n_wg / cus);
  const double w = std::max(1.0, per_cu * NW / 4.0);
  const double O = w < 1.5 ? 0.0 : w < 2.5 ? kOverlap2 : kOverlap3;
  const double tile = BC * D / 8.0 + kValuPer32 + 2.0 * BC * D / kLdsPerSimd - O + kKsFillPerD * D;
  const double hide = std::max(1.0, per_cu);
  const double pro = kKsPrologue + (32.0 * D * 2.0 + 4.0 * BC * D) / kPrologueBytesPerCycle;
  std::vector<double> dur(n_qt);
  for (int t = 0; t < n_qt; ++t) {
    const int qt = s.causal ? n_qt - 1 - t : t;
    const int last = std::min(qt * 32 + 32, s.Sq) - 1;
    const int kv_end = s.causal ? std::max(0, std::min(s.Skv, last + off + 1)) : s.Skv;
    const int n_t = (kv_end + BC - 1) / BC;
    dur[t] = (n_t + NW - 1) / NW * tile + kKsMerge + (pro + kEpilogue) / hide;
  }
  const double machines_per_cu = NW >= 4 ? 1.0 : 4.0 / NW;
  const int64_t machines = std::max<int64_t>(1, (int64_t)(cus * machines_per_cu));
  std::priority_queue<double, std::vector<double>, std::greater<double>> freeat;
  for (int64_t m = 0; m < std::min<int64_t>(machines, n_wg); ++m) freeat.push(0.0);
  double makespan = 0.0;
  for (int t = 0; t < n_qt; ++t)
    for (int64_t j = 0; j < (int64_t)s.B * s.Hq; ++j) {
      const double t1 = freeat.top() + dur[t];
      freeat.pop();
      makespan = std::max(makespan, t1);
      freeat.push(t1);
    }
  return makespan / (kClockGHz * 1e3) + kLaunchUs;
}

double estimate_us(const Shape& s, Cand c, int occ, int cus) {
  if (c.split > 1 && c.split == c.nw) return estimate_ks_us(s, c.nw, occ, cus);
  const int D = s.d, NW = c.nw, BC = c.bc, SP = c.split, NQ = NW / SP, BR = 32 * NQ;
  const int off = s.Skv - s.Sq;
  const int n_qt = (s.Sq + BR - 1) / BR;
  const int64_t n_wg = (int64_t)n_qt * s.B * s.Hq;
  // Workgroups resident per compute unit: the occupancy, or fewer when the
  // grid is small; waves per SIMD from that.
  const double per_cu = std::min<double>(occ, (double)n_wg / cus);
  const double w = std::max(1.0, per_cu * NW / 4.0);
  const double k32 = BC / 32.0;
  const double M = BC * D / 8.0;
  const double V = kValuPer32 * k32;
  const double L = 4.0 * BC * D / kLdsPerSimd;
  const double O = (w < 1.5 ? 0.0 : w < 2.5 ? kOverlap2 : kOverlap3) * k32;
  const double busy_cost = M + V + L - O;
  // A key group's tile is moved by its NQ waves.
  const double wait_cost = kFillPerD * D / NQ * k32 + kSyncPerTile;
  const double hide = std::max(1.0, per_cu);
  const int step = NW > 4 ? 2 : 1;   // waves sharing one SIMD within a workgroup
  auto duration = [&](int qt) {
    const int q0 = qt * BR;
    const int last = std::min(q0 + BR, s.Sq) - 1;
    const int kv_end = s.causal ? std::min(s.Skv, last + off + 1) : s.Skv;
    const int n_t = (kv_end + BC - 1) / BC;
    const int n_steps = (n_t + SP - 1) / SP;   // every wave waits on every step
    double cyc = 0.0;
    for (int wv = 0; wv < NW; wv += step) {
      double simd = 0.0;
      for (int k = 0; k < step; ++k) {
        const int w = wv + k, qb = w % NQ, kg = w / NQ;
        const int r1 = std::min(q0 + 32 * qb + 31, s.Sq - 1);
        const int wk = s.causal ? std::max(0, std::min(s.Skv, r1 + off + 1)) : s.Skv;
        // The wave's tiles: kg, kg + SP, ... below its last key's tile.
        const int nt_w = std::min(n_t, (wk + BC - 1) / BC);
        const int busy = nt_w > kg ? (nt_w - kg + SP - 1) / SP : 0;
        simd += busy * busy_cost + n_steps * wait_cost;
      }
      cyc = std::max(cyc, simd);
    }
    const double pro = kPrologue + (BR * D * 2.0 + 4.0 * BC * D) / kPrologueBytesPerCycle;
    return cyc + (SP > 1 ? kSplitMerge : 0.0) + (pro + kEpilogue) / hide;
  };
  std::vector<double> dur(n_qt);
  for (int t = 0; t < n_qt; ++t) dur[t] = duration(s.causal ? n_qt - 1 - t : t);
  const double machines_per_cu = NW >= 4 ? 1.0 : 4.0 / NW;
  const int64_t machines = std::max<int64_t>(1, (int64_t)(cus * machines_per_cu));
  std::priority_queue<double, std::vector<double>, std::greater<double>> freeat;
  for (int64_t m = 0; m < std::min<int64_t>(machines, n_wg); ++m) freeat.push(0.0);
  double makespan = 0.0;
  const int64_t per_t = (int64_t)s.B * s.Hq;
  for (int t = 0; t < n_qt; ++t) {
    for (int64_t j = 0; j < per_t; ++j) {
      const double t1 = freeat.top() + dur[t];
      freeat.pop();
      makespan = std::max(makespan, t1);
      freeat.push(t1);
    }
  }
  return makespan / (kClockGHz * 1e3) + kLaunchUs;
}

struct KeyHash {
  size_t operator()(const std::vector<int>& k) const {
    size_t h = 1469598103934665603ull;
    for (int x : k) h = (h ^ (size_t)(unsigned)x) * 1099511628211ull;
    return h;
  }
};

thread_local int t_override_nw = 0, t_override_bc = 0, t_override_split = 0;

int device_cus_cached() {
  static int cus = 0;
  if (!cus) cus = device_cus();
  return cus;
}

}  // namespace

int fwd_tile_plan(int d, int causal, int B, int Hq, int Hkv, int Sq, int Skv, int cap, int* nw,
                  int* bc, int* split, float* est_us, int* pick) {
  const Cand* cs = nullptr;
  const int n = candidates(d, &cs);
  if (!n) return 0;
  const Shape s{d, causal ? 1 : 0, B, Hq, Hkv, Sq, Skv};
  const int cus = device_cus_cached();
  int best = 0;
  double best_t = 0.0;
  for (int i = 0; i < n; ++i) {
    const double t = estimate_us(s, cs[i], occupancy(d, causal != 0, i, cs[i].nw), cus);
    if (i < cap) {
      if (nw) nw[i] = cs[i].nw;
      if (bc) bc[i] = cs[i].bc;
      if (split) split[i] = cs[i].split;
      if (est_us) est_us[i] = (float)t;
    }
    if (i == 0 || t < best_t) {
      best = i;
      best_t = t;
    }
  }
  if (pick) *pick = best;
  return n;
}

bool fwd_tile_override_ok(int d) {
  if (!t_override_nw) return true;
  const Cand* cs = nullptr;
  const int n = candidates(d, &cs);
  for (int i = 0; i < n; ++i)
    if (cs[i].nw == t_override_nw && cs[i].bc == t_override_bc &&
        cs[i].split == t_override_split)
      return true;
  return false;
}

void fwd_tile_set_override(int nw, int bc, int split) {
  t_override_nw = nw;
  t_override_bc = bc;
  t_override_split = split;
}

int fwd_pick_candidate(const FwdArgs& a) {
  const Cand* cs = nullptr;
  const int n = candidates(a.d, &cs);
  if (t_override_nw) {
    for (int i = 0; i < n; ++i)
      if (cs[i].nw == t_override_nw && cs[i].bc == t_override_bc &&
          cs[i].split == t_override_split)
        return i;
  }
  static std::mutex mu;
  static std::unordered_map<std::vector<int>, int, KeyHash> cache;
  int dev = 0;
  (void)hipGetDevice(&dev);
  const std::vector<int> key{dev, a.d, a.causal, a.B, a.Hq, a.Hkv, a.Sq, a.Skv};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int pick = 0;
  fwd_tile_plan(a.d, a.causal, a.B, a.Hq, a.Hkv, a.Sq, a.Skv, 0, nullptr, nullptr, nullptr,
                nullptr, &pick);
  std::lock_guard<std::mutex> lock(mu);
  if (cache.size() > 4096) cache.clear();
  cache[key] = pick;
  return pick;
}

}  // namespace attn
