// C ABI of libattn.so: argument validation and dispatch.  Every check runs
// on the host before anything is enqueued, so a rejected call launches
// nothing ("Compilers and Kernels", section "A kernel implements a bounded
// contract": a specialised kernel must guard shape, stride, dtype, layout
// and aliasing facts or keep a general path; this library guards them and
// reports an error instead of guessing).
#include "../../include/attn.h"

#include <math.h>

#include <algorithm>
#include <stdint.h>

#include <mutex>

#include "launch.h"

namespace {

constexpr int kAbiVersion = 5;
constexpr int kMaxSplits = 256;

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + (uintptr_t)bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int esize(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool dtype_ok(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_BF16; }

bool fwd_d_ok(int dtype, int d) { return dtype_ok(dtype) && (d == 64 || d == 128 || d == 256); }
bool decode_d_ok(int dtype, int d) { return dtype_ok(dtype) && (d == 64 || d == 128 || d == 256); }
bool bwd_d_ok(int dtype, int d) { return dtype == ATTN_BF16 && (d == 64 || d == 128 || d == 256); }
bool bwd_fused_d_ok(int dtype, int d) { return dtype == ATTN_BF16 && (d == 64 || d == 128); }
bool paged_d_ok(int dtype, int d) { return dtype == ATTN_BF16 && (d == 64 || d == 128); }

// Per-head element counts must stay within 32-bit index arithmetic.
bool sizes_ok(int64_t S, int d) { return S * (int64_t)d < (int64_t(1) << 31); }

// An additive bias: 16-byte aligned rows (Skv and both strides multiples
// of 4 floats), non-negative strides; on success *extent is its byte span.
attn_status check_bias(const float* bias, int64_t sb, int64_t sh, int B, int Hq, int Sq, int Skv,
                       int64_t* extent) {
  *extent = 0;
  if (!bias) return ATTN_OK;
  if (sb < 0 || sh < 0) return ATTN_ERR_VALUE;
  if (!aligned16(bias) || Skv % 4 != 0 || sb % 4 != 0 || sh % 4 != 0) return ATTN_ERR_ALIGN;
  const int64_t last = (int64_t)(B - 1) * sb + (int64_t)(Hq - 1) * sh + (int64_t)Sq * Skv;
  if (last >= (int64_t(1) << 60) / 4) return ATTN_ERR_SHAPE;
  *extent = last * 4;
  return ATTN_OK;
}

// Outputs must not overlap inputs or each other.
attn_status check_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    if (outs[i].lo == outs[i].hi) continue;
    for (int j = 0; j < n_in; ++j)
      if (ins[j].lo != ins[j].hi && overlap(outs[i], ins[j])) return ATTN_ERR_ALIAS;
    for (int j = i + 1; j < n_out; ++j)
      if (outs[j].lo != outs[j].hi && overlap(outs[i], outs[j])) return ATTN_ERR_ALIAS;
  }
  return ATTN_OK;
}

attn_status hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

thread_local void* const* g_events = nullptr;
thread_local int g_n_events = 0;

}  // namespace

namespace attn {
static thread_local int t_dkdv_nkw = 0, t_dkdv_hs = 0, t_dq_nqw = 0, t_dq_hs = 0,
                        t_hsplit = 0;
void bwd_set_tile_override(int nkw, int hs, int nqw, int qhs, int hsplit) {
  t_dkdv_nkw = nkw;
  t_dkdv_hs = hs;
  t_dq_nqw = nqw;
  t_dq_hs = qhs;
  t_hsplit = hsplit;
}

// The three shapes' estimated times from the grid's load per compute unit
// and its longest workgroup (see bwd_dkdv_config): the plain shape's
// workgroups run two per compute unit, and a heavy one may end alone on
// its compute unit at one wave per SIMD (chain41 units per iteration);
// (4, 2) halves a workgroup's iterations over two groups at two waves per
// SIMD; (2, 4) quarters them over twice as many workgroups.  ovh42 and
// ovh24 price the grouped shapes' merge and extra loads.  Ties go to the
// plain shape.  Returns the pick as (blocks per workgroup, groups).
static void pick_shape(double load, double n_max, double chain41, double ovh42, double ovh24,
                       int* nb, int* hs) {
  const double t41 = std::max(load, chain41 * n_max);
  const double t42 = std::max(ovh42 * load, n_max);
  const double t24 = std::max(ovh24 * load, 0.5 * n_max);
  *nb = 4;
  *hs = 1;
  if (t42 < t41 && t42 <= t24) {
    *hs = 2;
  } else if (t24 < t41 && t24 < t42) {
    *nb = 2;
    *hs = 4;
  }
}

void bwd_dq_config(const BwdArgs& a, int* nqw, int* hs) {
  if (t_dq_nqw) {
    *nqw = t_dq_nqw;
    *hs = t_dq_hs;
    return;
  }
  // Per 128-row workgroup the iterations are its 32-key blocks: the keys up
  // to its last row's causal bound, from its first row's window start.
  const int off = a.Skv - a.Sq;
  const bool win = a.causal && a.window > 0;
  const int nq = (a.Sq + 127) / 128;
  double sum = 0.0;
  int nb_max = 0;
  for (int qt = 0; qt < nq; ++qt) {
    const int last = std::min(qt * 128 + 127, a.Sq - 1);
    const int kv_end = a.causal ? std::min(a.Skv, last + off + 1) : a.Skv;
    const int kv_begin = win ? std::max(0, qt * 128 + off - a.window + 1) / 32 * 32 : 0;
    const int nb = std::max(0, (kv_end - kv_begin + 31) / 32);
    sum += nb;
    nb_max = std::max(nb_max, nb);
  }
  // Fitted on MI355X: the plain dQ kernel's heavy workgroups run at about
  // one unit per iteration even alone on a compute unit (chain 1.0), and the
  // grouped shapes' 32-key tiles (the plain kernel's are 64) cost 15 % at
  // (4, 2) and 40 % at (2, 4).
  const double load = sum * a.B * a.Hq / device_cus();
  pick_shape(load, (double)nb_max, 1.0, 1.15, 1.40, nqw, hs);
}
int64_t bwd_split_part_offset(int B, int Hq, int Sq) {
  const int64_t sqp = ((int64_t)Sq + 31) / 32 * 32;
  return (2 * (int64_t)B * Hq * sqp + 63) / 64 * 64;   // the pairs, rounded to 256 bytes
}

size_t bwd_split_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int d, int p) {
  const size_t pairs = ((size_t)bwd_split_part_offset(B, Hq, Sq)) * sizeof(float);
  if (p <= 1) return pairs;
  return round256(pairs + (size_t)p * 2 * B * Hkv * Skv * d * sizeof(float));
}

void bwd_dkdv_config(const BwdArgs& a, int* nkw, int* hs, int* hsplit) {
  const bool plain = a.window == 0 && !a.bias;
  auto fits = [&](int p) {
    return a.ws_bytes >= bwd_split_workspace_bytes(a.B, a.Hq, a.Hkv, a.Sq, a.Skv, a.d, p);
  };
  // A forced shape or split (attn_bwd_tile_override) is taken as it is; a
  // forced split the workspace cannot hold is reported by attn_bwd.  d = 256
  // has only the plain shape; masked calls do not split.
  const int forced_p = plain ? t_hsplit : (t_hsplit ? 1 : 0);
  const bool forced_shape = t_dkdv_nkw != 0 && a.d <= 128;
  *nkw = forced_shape ? t_dkdv_nkw : 4;
  *hs = forced_shape ? t_dkdv_hs : 1;
  *hsplit = forced_p ? forced_p : 1;
  if ((forced_shape || a.d > 128) && forced_p) return;
  // Estimated time of each launch, in units of one wave's pass over one
  // query iteration (query head, 32-row query tile) of its 32-key block:
  // the larger of the grid's load per compute unit and the longest
  // workgroup.  Per 128 keys the iterations are the query tiles that can
  // see those keys (causal and window bounds, as in the kernel) times the
  // G query heads of the key/value head.  The load is their sum over the
  // 128-key workgroups divided by the compute units (two waves share each
  // SIMD in every shape).  The longest workgroup, n_max iterations: about
  // 1.3 n_max for the plain kernel (its heavy workgroups end up alone on a
  // compute unit, one wave per SIMD), n_max for (4, 2) (two groups, two
  // waves per SIMD), n_max / 2 for (2, 4).  The grouped shapes pay for the
  // merge and, with 64 keys per workgroup, for loading every Q / dO tile
  // twice as often: 5 % for (4, 2); for (2, 4) 5 % with grouped heads and
  // 40 % without (measured on MI355X: short iteration lists amortise the
  // per-workgroup costs worst).  At d = 256 only the plain shape exists,
  // one wave per SIMD, whose long chains run at about 0.75 load units per
  // iteration.
  //   At d <= 128 a tail of 0.1 times the longest workgroup's chain is
  //   added: the last workgroups leave compute units idle, and the grids
  //   with shorter workgroups measure faster even where the load bounds
  //   them.  A head split over p workgroups per key tile divides n_max by
  //   p (each takes every p-th query head) and adds its float32 partials:
  //   their writes hide under the kernel's arithmetic, the reduce reads
  //   them back (8 p bytes per dK/dV element) at about 5.5 TB/s, plus its
  //   launch; a unit is about 1.15 d/128 us (d <= 128) or 2.9 us (d = 256)
  //   to weigh them.  Ties go to the plain kernel and to fewer shares.
  const int G = a.Hq / a.Hkv;
  const int off = a.causal ? a.Skv - a.Sq : a.Skv;
  const bool win = a.causal && a.window > 0;
  const int nk = (a.Skv + 127) / 128;
  double sum = 0.0;
  int nq_max = 0;
  for (int kt = 0; kt < nk; ++kt) {
    const int q_start = a.causal ? (std::max(0, kt * 128 - off) / 32) * 32 : 0;
    const int q_end = win ? std::min(a.Sq, kt * 128 + 127 - off + a.window) : a.Sq;
    const int nq = std::max(0, (q_end - q_start + 31) / 32);
    sum += nq;
    nq_max = std::max(nq_max, nq);
  }
  const double load = sum * a.B * a.Hkv * G / device_cus();
  const double unit_us = a.d > 128 ? 2.9 : 1.15 * a.d / 128.0;
  const double nkv = (double)a.B * a.Hkv * a.Skv * a.d;
  const double tail = a.d > 128 ? 0.0 : 0.1;
  double best = INFINITY;
  for (int p = 1; p <= 8; p *= 2) {
    if (forced_p && p != forced_p) continue;
    if (!forced_p && p > 1 && (!plain || p > G || !fits(p))) break;
    const double gl = std::ceil((double)G / p);   // query heads per workgroup
    const double n_max = gl * nq_max;
    const double extra = p > 1 ? (3.0 + 8.0 * p * nkv / 5.5e6) / unit_us : 0.0;
    struct Shape { int nkw, hs; double ovh, chain; };
    const Shape shapes[3] = {{4, 1, 1.0, a.d > 128 ? 0.75 : 1.3},
                             {4, 2, 1.05, 1.0},
                             {2, 4, gl > 1 ? 1.05 : 1.40, 0.5}};
    for (int si = 0; si < (a.d > 128 ? 1 : 3); ++si) {
      const Shape& sh = shapes[si];
      if (forced_shape && (sh.nkw != t_dkdv_nkw || sh.hs != t_dkdv_hs)) continue;
      const double t = std::max(sh.ovh * load, sh.chain * n_max) + tail * sh.chain * n_max + extra;
      if (t < best * 0.999) {
        best = t;
        *nkw = sh.nkw;
        *hs = sh.hs;
        *hsplit = p;
      }
    }
  }
}

void timing_events(int i, hipEvent_t* start, hipEvent_t* stop) {
  *start = (g_events && 2 * i < g_n_events) ? (hipEvent_t)g_events[2 * i] : nullptr;
  *stop = (g_events && 2 * i + 1 < g_n_events) ? (hipEvent_t)g_events[2 * i + 1] : nullptr;
}
}  // namespace attn

extern "C" {

int attn_abi_version(void) { return kAbiVersion; }

const char* attn_status_str(int s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (non-positive size, Hq % Hkv != 0, causal with Sq > Skv, or too large)";
    case ATTN_ERR_UNSUPPORTED: return "head dim or dtype not compiled for this entry point";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_ALIAS: return "an output overlaps an input or another output";
    case ATTN_ERR_WORKSPACE:
      return "workspace missing or too small (attn_decode_noalloc: the split states need more "
             "than the library's static scratch of ATTN_SCRATCH_BYTES bytes)";
    case ATTN_ERR_HIP: return "HIP launch failed";
    case ATTN_ERR_VALUE: return "invalid scalar argument (scale not finite or n_splits out of range)";
  }
  return "unknown status";
}

attn_status attn_fwd_tile_override(int nw, int bc, int split) {
  const bool none = nw == 0 && bc == 0 && split == 0;
  if (!none && (nw <= 0 || bc <= 0 || split <= 0 || nw % split != 0)) return ATTN_ERR_VALUE;
  attn::fwd_tile_set_override(nw, bc, split);
  return ATTN_OK;
}

attn_status attn_bwd_tile_override(int nkw, int hs, int nqw, int qhs, int hsplit) {
  auto ok = [](int nb, int h) {
    return (nb == 0 && h == 0) || (nb == 4 && h == 1) || (nb == 4 && h == 2) || (nb == 2 && h == 4);
  };
  if (!ok(nkw, hs) || !ok(nqw, qhs) || hsplit < 0 || hsplit > 8) return ATTN_ERR_VALUE;
  attn::bwd_set_tile_override(nkw, hs, nqw, qhs, hsplit);
  return ATTN_OK;
}

int attn_fwd_tile_plan(int d, int causal, int B, int Hq, int Hkv, int Sq, int Skv, int cap,
                       int* nw, int* bc, int* split, float* est_us, int* pick) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || Hq % Hkv != 0 || cap < 0)
    return 0;
  if (causal && Sq > Skv) return 0;
  return attn::fwd_tile_plan(d, causal, B, Hq, Hkv, Sq, Skv, cap, nw, bc, split, est_us, pick);
}

attn_status attn_set_timing_events(void* const* events, int n) {
  if (n < 0) return ATTN_ERR_VALUE;
  g_events = (events && n > 0) ? events : nullptr;
  g_n_events = g_events ? n : 0;
  return ATTN_OK;
}

int attn_supports(int dtype, int entry, int d) {
  switch (entry) {
    case 0: return fwd_d_ok(dtype, d);
    case 1: return decode_d_ok(dtype, d);
    case 2: return bwd_d_ok(dtype, d);
    case 3: return paged_d_ok(dtype, d);
    case 4: return bwd_fused_d_ok(dtype, d);
  }
  return 0;
}

attn_status attn_fwd(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d, int causal, int window,
                     const float* bias, int64_t bias_sb, int64_t bias_sh, float scale,
                     void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal && Sq > Skv) return ATTN_ERR_SHAPE;
  if (window > 0 && !causal) return ATTN_ERR_VALUE;
  if (!sizes_ok(Sq, d) || !sizes_ok(Skv, d)) return ATTN_ERR_SHAPE;
  if (!fwd_d_ok(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  // A forced tile shape (attn_fwd_tile_override) must be compiled for d.
  if (dtype == ATTN_BF16 && !attn::fwd_tile_override_ok(d)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  int64_t bias_bytes = 0;
  attn_status st = check_bias(bias, bias_sb, bias_sh, B, Hq, Sq, Skv, &bias_bytes);
  if (st != ATTN_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_ERR_ALIGN;
  const int es = esize(dtype);
  const Span ins[4] = {span(q, (int64_t)B * Hq * Sq * d * es), span(k, (int64_t)B * Hkv * Skv * d * es),
                       span(v, (int64_t)B * Hkv * Skv * d * es), span(bias, bias_bytes)};
  const Span outs[2] = {span(o, (int64_t)B * Hq * Sq * d * es),
                        lse ? span(lse, (int64_t)B * Hq * Sq * 4) : Span{0, 0}};
  st = check_alias(outs, 2, ins, 4);
  if (st != ATTN_OK) return st;
  attn::FwdArgs a{dtype, q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, causal ? 1 : 0,
                  window > 0 && window < Skv ? window : 0, bias, bias_sb, bias_sh, scale,
                  (hipStream_t)stream};
  return hip_status(attn::launch_fwd(a));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int d, int n_splits) {
  if (B <= 0 || Hq <= 0 || d <= 0 || n_splits <= 0) return 0;
  return round256((size_t)n_splits * B * Hq * (size_t)(d + 2) * sizeof(float));
}

}  // extern "C"

namespace {

// Argument checks shared by attn_decode and attn_decode_noalloc (which has
// no caller workspace: check_ws false leaves the workspace out).
attn_status check_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                         void* o, float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                         int n_splits, void* workspace, size_t workspace_bytes,
                         bool check_ws = true) {
  if (!q || !k_cache || !v_cache || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Skv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!sizes_ok(Skv, d)) return ATTN_ERR_SHAPE;
  if (!decode_d_ok(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  if (n_splits < 1 || n_splits > kMaxSplits) return ATTN_ERR_VALUE;
  if (check_ws) {
    if (!workspace) return ATTN_ERR_WORKSPACE;
    if (workspace_bytes < attn_decode_workspace_bytes(B, Hq, d, n_splits))
      return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  }
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      (lse && !aligned16(lse)))
    return ATTN_ERR_ALIGN;
  const int es = esize(dtype);
  const Span ins[3] = {span(q, (int64_t)B * Hq * d * es),
                       span(k_cache, (int64_t)B * Hkv * Skv * d * es),
                       span(v_cache, (int64_t)B * Hkv * Skv * d * es)};
  const Span outs[3] = {span(o, (int64_t)B * Hq * d * es),
                        lse ? span(lse, (int64_t)B * Hq * 4) : Span{0, 0},
                        check_ws ? span(workspace, (int64_t)attn_decode_workspace_bytes(
                                                       B, Hq, d, n_splits))
                                 : Span{0, 0}};
  return check_alias(outs, 3, ins, 3);
}

}  // namespace

extern "C" {

attn_status attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache, void* o,
                        float* lse, int B, int Hq, int Hkv, int Skv, int d, float scale,
                        int n_splits, void* workspace, size_t workspace_bytes, void* stream) {
  const attn_status st = check_decode(dtype, q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d,
                                      scale, n_splits, workspace, workspace_bytes);
  if (st != ATTN_OK) return st;
  attn::DecodeArgs a{dtype, q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, n_splits, scale,
                     (float*)workspace, (hipStream_t)stream};
  return hip_status(attn::launch_decode(a));
}

attn_status attn_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                              const int* block_table, const int* seq_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int d, int n_pages, int page_size,
                              int max_pages, float scale, int n_splits, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !o) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || n_pages <= 0 || page_size <= 0 ||
      max_pages <= 0)
    return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (!paged_d_ok(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  if (page_size % 32 != 0) return ATTN_ERR_VALUE;
  // Keys per stream and elements per page stay in 32-bit index arithmetic.
  if ((int64_t)max_pages * page_size >= (int64_t(1) << 31) || !sizes_ok(page_size, d))
    return ATTN_ERR_SHAPE;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  if (n_splits < 1 || n_splits > kMaxSplits) return ATTN_ERR_VALUE;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_decode_workspace_bytes(B, Hq, d, n_splits)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(o) ||
      (lse && !aligned16(lse)) || !aligned16(workspace) || !aligned4(block_table) ||
      !aligned4(seq_lens))
    return ATTN_ERR_ALIGN;
  const int es = esize(dtype);
  const int64_t pool = (int64_t)n_pages * Hkv * page_size * d * es;
  const Span ins[5] = {span(q, (int64_t)B * Hq * d * es), span(k_pages, pool),
                       span(v_pages, pool), span(block_table, (int64_t)B * max_pages * 4),
                       span(seq_lens, (int64_t)B * 4)};
  const Span outs[3] = {span(o, (int64_t)B * Hq * d * es),
                        lse ? span(lse, (int64_t)B * Hq * 4) : Span{0, 0},
                        span(workspace, (int64_t)attn_decode_workspace_bytes(B, Hq, d, n_splits))};
  attn_status st = check_alias(outs, 3, ins, 5);
  if (st != ATTN_OK) return st;
  attn::DecodeArgs a{dtype, q, k_pages, v_pages, o, lse, B, Hq, Hkv, 0, d, n_splits, scale,
                     (float*)workspace, (hipStream_t)stream,
                     attn::PagedKV{block_table, seq_lens, max_pages, page_size, n_pages}};
  return hip_status(attn::launch_decode(a));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Static scratch for attn_decode_noalloc: the split states live in this
// array instead of a caller's workspace.  Every device the library runs on
// holds its own copy for the life of the process.  On the host, `scratch`
// only names the symbol; its device address (one per device) comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------
namespace {

static __device__ __align__(256) unsigned char scratch[ATTN_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device), or an error.
attn_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_decode_noalloc(int dtype, const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse, int B, int Hq, int Hkv,
                                int Skv, int d, float scale, int n_splits, void* stream) {
  // A problem whose split states exceed the static array is rejected before
  // anything is enqueued.
  if (attn_decode_workspace_bytes(B, Hq, d, n_splits) > ATTN_SCRATCH_BYTES)
    return ATTN_ERR_WORKSPACE;
  attn_status st = check_decode(dtype, q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, scale,
                                n_splits, nullptr, 0, false);
  if (st != ATTN_OK) return st;
  void* ws = nullptr;
  st = scratch_ptr(&ws);
  if (st != ATTN_OK) return st;
  attn::DecodeArgs a{dtype, q, k_cache, v_cache, o, lse, B, Hq, Hkv, Skv, d, n_splits, scale,
                     (float*)ws, (hipStream_t)stream};
  return hip_status(attn::launch_decode(a));
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Sq, int d) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || d <= 0) return 0;
  const size_t sqp = ((size_t)Sq + 31) / 32 * 32;
  return round256(2 * (size_t)B * Hq * sqp * sizeof(float));
}

attn_status attn_bwd(int dtype, const void* q, const void* k, const void* v, const void* o,
                     const void* d_o, const float* lse, void* dq, void* dk, void* dv, int B,
                     int Hq, int Hkv, int Sq, int Skv, int d, int causal, int window,
                     const float* bias, int64_t bias_sb, int64_t bias_sh, float scale,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal && Sq > Skv) return ATTN_ERR_SHAPE;
  if (window > 0 && !causal) return ATTN_ERR_VALUE;
  if (!sizes_ok(Sq, d) || !sizes_ok(Skv, d)) return ATTN_ERR_SHAPE;
  // The kernels address the workspace with 32-bit byte offsets.
  if (attn_bwd_workspace_bytes(B, Hq, Sq, d) > 0xffffffffu) return ATTN_ERR_SHAPE;
  if (!bwd_d_ok(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  int64_t bias_bytes = 0;
  attn_status st = check_bias(bias, bias_sb, bias_sh, B, Hq, Sq, Skv, &bias_bytes);
  if (st != ATTN_OK) return st;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, Hq, Sq, d)) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return ATTN_ERR_ALIGN;
  attn::BwdArgs a{dtype, q, k, v, o, d_o, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, d,
                  causal ? 1 : 0, window > 0 && window < Skv ? window : 0, bias, bias_sb, bias_sh, scale,
                  (float*)workspace, (hipStream_t)stream, workspace_bytes};
  // The workspace the call will use: the pairs, plus the head split's
  // partials when it splits (the split it picks fits the workspace given;
  // a forced one that does not is an error).
  int nkw = 4, hs = 1, hsplit = 1;
  if (d <= 256) attn::bwd_dkdv_config(a, &nkw, &hs, &hsplit);
  const size_t ws_used = attn::bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, hsplit);
  if (workspace_bytes < ws_used) return ATTN_ERR_WORKSPACE;
  const int es = esize(dtype);
  const int64_t nq = (int64_t)B * Hq * Sq * d * es, nkv = (int64_t)B * Hkv * Skv * d * es;
  const Span ins[7] = {span(q, nq), span(k, nkv), span(v, nkv), span(o, nq), span(d_o, nq),
                       span(lse, (int64_t)B * Hq * Sq * 4), span(bias, bias_bytes)};
  const Span outs[4] = {span(dq, nq), span(dk, nkv), span(dv, nkv),
                        span(workspace, (int64_t)ws_used)};
  st = check_alias(outs, 4, ins, 7);
  if (st != ATTN_OK) return st;
  return hip_status(attn::launch_bwd(a));
}

size_t attn_bwd_split_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int d,
                                      int causal) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0 || Hq % Hkv != 0) return 0;
  if (causal && Sq > Skv) return 0;
  attn::BwdArgs a{ATTN_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, B, Hq, Hkv, Sq, Skv, d, causal ? 1 : 0, 0, nullptr, 0, 0,
                  1.f, nullptr, nullptr, (size_t)-1};
  int nkw = 4, hs = 1, hsplit = 1;
  attn::bwd_dkdv_config(a, &nkw, &hs, &hsplit);
  return attn::bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, hsplit);
}

attn_status attn_bwd_plan(int B, int Hq, int Hkv, int Sq, int Skv, int d, int causal, int window,
                          int has_bias, size_t workspace_bytes, int* nkw, int* hs, int* nqw,
                          int* qhs, int* hsplit) {
  if (!nkw || !hs || !nqw || !qhs || !hsplit) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal && Sq > Skv) return ATTN_ERR_SHAPE;
  if (window > 0 && !causal) return ATTN_ERR_VALUE;
  if (!sizes_ok(Sq, d) || !sizes_ok(Skv, d)) return ATTN_ERR_SHAPE;
  if (attn_bwd_workspace_bytes(B, Hq, Sq, d) > 0xffffffffu) return ATTN_ERR_SHAPE;
  if (!bwd_d_ok(ATTN_BF16, d)) return ATTN_ERR_UNSUPPORTED;
  if (workspace_bytes < attn_bwd_workspace_bytes(B, Hq, Sq, d)) return ATTN_ERR_WORKSPACE;
  // Only whether a bias is given matters to the plan, never its values.
  static const float no_values = 0.f;
  attn::BwdArgs a{ATTN_BF16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                  nullptr, nullptr, B, Hq, Hkv, Sq, Skv, d, causal ? 1 : 0,
                  window > 0 && window < Skv ? window : 0, has_bias ? &no_values : nullptr, 0, 0,
                  1.f, nullptr, nullptr, workspace_bytes};
  attn::bwd_dkdv_config(a, nkw, hs, hsplit);
  if (d <= 128) {
    attn::bwd_dq_config(a, nqw, qhs);
  } else {
    *nkw = 4;
    *hs = 1;
    *nqw = 4;
    *qhs = 1;
  }
  if (workspace_bytes < attn::bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, *hsplit))
    return ATTN_ERR_WORKSPACE;
  return ATTN_OK;
}

size_t attn_bwd_fused_workspace_bytes(int B, int Hq, int Sq, int d) {
  if (B <= 0 || Hq <= 0 || Sq <= 0 || d <= 0) return 0;
  return round256((size_t)attn::bwd_fused_acc_offset(B, Hq, Sq) * sizeof(float) +
                  (size_t)B * Hq * Sq * d * sizeof(float));
}

attn_status attn_bwd_fused(int dtype, const void* q, const void* k, const void* v, const void* o,
                           const void* d_o, const float* lse, void* dq, void* dk, void* dv, int B,
                           int Hq, int Hkv, int Sq, int Skv, int d, int causal, int window,
                           const float* bias, int64_t bias_sb, int64_t bias_sh, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || d <= 0) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (causal && Sq > Skv) return ATTN_ERR_SHAPE;
  if (window > 0 && !causal) return ATTN_ERR_VALUE;
  if (!sizes_ok(Sq, d) || !sizes_ok(Skv, d)) return ATTN_ERR_SHAPE;
  // The (D, nl) pairs are addressed with 32-bit byte offsets.
  if (attn_bwd_workspace_bytes(B, Hq, Sq, d) > 0xffffffffu) return ATTN_ERR_SHAPE;
  if (!bwd_fused_d_ok(dtype, d)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_VALUE;
  int64_t bias_bytes = 0;
  attn_status st = check_bias(bias, bias_sb, bias_sh, B, Hq, Sq, Skv, &bias_bytes);
  if (st != ATTN_OK) return st;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  const size_t ws_need = attn_bwd_fused_workspace_bytes(B, Hq, Sq, d);
  if (workspace_bytes < ws_need) return ATTN_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(d_o) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return ATTN_ERR_ALIGN;
  const int es = esize(dtype);
  const int64_t nq = (int64_t)B * Hq * Sq * d * es, nkv = (int64_t)B * Hkv * Skv * d * es;
  const Span ins[7] = {span(q, nq), span(k, nkv), span(v, nkv), span(o, nq), span(d_o, nq),
                       span(lse, (int64_t)B * Hq * Sq * 4), span(bias, bias_bytes)};
  const Span outs[4] = {span(dq, nq), span(dk, nkv), span(dv, nkv),
                        span(workspace, (int64_t)ws_need)};
  st = check_alias(outs, 4, ins, 7);
  if (st != ATTN_OK) return st;
  attn::BwdArgs a{dtype, q, k, v, o, d_o, lse, dq, dk, dv, B, Hq, Hkv, Sq, Skv, d,
                  causal ? 1 : 0, window > 0 && window < Skv ? window : 0, bias, bias_sb, bias_sh,
                  scale, (float*)workspace, (hipStream_t)stream};
  return hip_status(attn::launch_bwd_fused(a));
}

}  // extern "C"
