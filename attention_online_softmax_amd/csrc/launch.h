// Host-side launch descriptors passed from the C ABI layer to the kernel
// launchers.  Arguments are validated before any of these is filled in.
#pragma once

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
  float* ws;  // [B, Hq, Sqp] pairs (D = rowsum(dO * O), -LSE * log2(e)); Sqp = Sq rounded up to 32
  hipStream_t stream;
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

// Records the caller's timing event for `slot` (2i before / 2i+1 after the
// i-th kernel of the current entry point) if timing events are set.
void timing_mark(hipStream_t stream, int slot);

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
hipError_t launch_bwd_d256(const BwdArgs& a);   // d = 256 (bwd256.hip)
// Fused variant (no window or bias): ws holds the (D, nl) pairs, then from
// bwd_fused_acc_offset floats on the fp32 dQ accumulator [B, Hq, Sq, d].
hipError_t launch_bwd_fused(const BwdArgs& a);
int64_t bwd_fused_acc_offset(int B, int Hq, int Sq);
// The fused dK/dV/dQ kernel alone (a.ws holds the pairs; dqacc is cleared).
hipError_t launch_dkdv_fused(const BwdArgs& a, float* dqacc);

}  // namespace attn
