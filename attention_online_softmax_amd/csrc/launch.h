// Host-side launch descriptors passed from the C ABI layer to the kernel
// launchers.  Arguments are validated before any of these is filled in.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdArgs {
  int dtype;  // 0 = f32, 1 = bf16
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Sq, Skv, d, causal;
  int window;  // sliding-window width (causal only), 0 = none
  const float* bias;  // additive mask bias[b*bias_sb + h*bias_sh + i*Skv + j], or nullptr
  int64_t bias_sb, bias_sh;
  float scale;
  hipStream_t stream;
};

// Paged key/value cache: pools [n_pages, Hkv, page_size, d], a block table
// [B, max_pages] of page ids and per-stream lengths [B], both in device
// memory (table == nullptr: contiguous caches).
struct PagedKV {
  const int* table;
  const int* lens;
  int max_pages, page_size, n_pages;
};

struct DecodeArgs {
  int dtype;
  const void* q;
  const void* k;  // [B, Hkv, Skv, d], or the key pool when paged
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Skv, d, n_splits;  // Skv unused when paged
  float scale;
  float* ws;  // [n_splits, B, Hq] m, then l, then [n_splits, B, Hq, d] acc
  hipStream_t stream;
  PagedKV pg;  // table == nullptr for contiguous caches
};

struct BwdArgs {
  int dtype;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, Sq, Skv, d, causal;
  int window;  // sliding-window width (causal only), 0 = none
  const float* bias;  // as in FwdArgs
  int64_t bias_sb, bias_sh;
  float scale;
  float* ws;  // [B, Hq, Sqp] pairs (D = rowsum(dO * O), -LSE * log2(e)); Sqp = Sq rounded up to 32,
              // then (head split) float32 dK/dV partials
  hipStream_t stream;
  size_t ws_bytes = 0;  // the workspace's size (attn_bwd): bounds the head split
};

// Compute units of the current device (256 if the query fails).
inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

// The caller's timing events for the i-th kernel of the current entry point
// (slots 2i and 2i + 1; null where none is set).
void timing_events(int i, hipEvent_t* start, hipEvent_t* stop);

hipError_t launch_fwd(const FwdArgs& a);
// bf16 forward tile selection (fwd_tiles.cpp): index of the compiled
// candidate (waves per workgroup, keys per tile) for a plain call; the
// per-candidate estimates; a per-thread override for sweeps and tests.
int fwd_pick_candidate(const FwdArgs& a);
int fwd_tile_plan(int d, int causal, int B, int Hq, int Hkv, int Sq, int Skv, int cap, int* nw,
                  int* bc, int* split, float* est_us, int* pick);
bool fwd_tile_override_ok(int d);
void fwd_tile_set_override(int nw, int bc, int split);
hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
// dK/dV launch shape of a call at d <= 128: key blocks of 32 per workgroup
// (nkw) and wave groups that split the query iterations (hs): (4, 1), or
// (4, 2) / (2, 4) on grids of fewer 128-key workgroups than compute units;
// and a per-thread override for sweeps and tests ((0, 0) = none).
void bwd_dkdv_config(const BwdArgs& a, int* nkw, int* hs, int* hsplit);
// Head split of the dK/dV kernel (plain calls): float32 partials of dK and
// dV per share of the query heads, at this offset (floats) in the backward
// workspace: [hsplit][2][B, Hkv, Skv, d].  The workspace for a split of p.
int64_t bwd_split_part_offset(int B, int Hq, int Sq);
size_t bwd_split_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int d, int p);
// The same for the dQ kernel: 32-row query blocks per workgroup (nqw) and
// wave groups that split the key tiles (hs).
void bwd_dq_config(const BwdArgs& a, int* nqw, int* hs);
void bwd_set_tile_override(int nkw, int hs, int nqw, int qhs, int hsplit);
hipError_t launch_bwd_d256(const BwdArgs& a);   // d = 256 (bwd256.hip)
// Fused variant (no window or bias): ws holds the (D, nl) pairs, then from
// bwd_fused_acc_offset floats on the fp32 dQ accumulator [B, Hq, Sq, d].
hipError_t launch_bwd_fused(const BwdArgs& a);
int64_t bwd_fused_acc_offset(int B, int Hq, int Sq);
// The fused dK/dV/dQ kernel alone (a.ws holds the pairs; dqacc is cleared).
hipError_t launch_dkdv_fused(const BwdArgs& a, float* dqacc);

}  // namespace attn

// Launch of the i-th kernel of an entry point.  While the caller has timing
// events set for it, they are bound to the launch itself (hipExtLaunchKernel
// records the kernel's start and end in them), so timing adds no packet of
// its own to the stream and no gap between kernels.
#define ATTN_LAUNCH(i, kernel, grid, block, stream, ...)                                \
  do {                                                                                  \
    hipEvent_t attn_e0_ = nullptr, attn_e1_ = nullptr;                                  \
    ::attn::timing_events((i), &attn_e0_, &attn_e1_);                                   \
    if (attn_e0_ || attn_e1_)                                                           \
      hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, attn_e0_, attn_e1_, 0,      \
                            __VA_ARGS__);                                               \
    else                                                                                \
      hipLaunchKernelGGL(kernel, grid, block, 0, stream, __VA_ARGS__);                  \
  } while (0)
