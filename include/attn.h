/*
 * attn.h -- C ABI of the online-softmax attention library (libattn.so).
 *
 * Computes scaled dot-product attention O = softmax(scale * Q K^T + C) V in
 * one pass over the keys, the way "Compilers and Kernels" (section
 * "FlashAttention changes the algorithm around IO") defines it: first display
 * equation for the function, second display equation for the blockwise
 * recurrence of running maximum m, normaliser l and accumulator o, and
 * O_i = o_T / l_T at the end.  Partial states over disjoint key ranges are
 * combined by the online-softmax monoid ("Tang, a compiler that derives GPU
 * kernels and bounds how fast they can run", Abstract): both sides are
 * rescaled to the larger maximum and added.  No score or probability matrix
 * is ever written to device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  q, k, v, o, lse and the gradient buffers are DEVICE pointers
 *   (memory from hipMalloc or a framework allocator on the current device).
 *   The caller owns every buffer, including workspaces; the library never
 *   allocates or frees device memory, keeps no state between calls and does
 *   not synchronise.  (One exception: attn_decode_noalloc keeps its split
 *   states in a static device array of the library, see there.)
 * Layout.  Dense, contiguous [B, H, S, d] (d innermost) for Q, K, V, O, dO,
 *   dQ, dK, dV; [B, Hq, Sq] float32 for LSE.  K and V share Hkv heads; query
 *   head h reads key/value head h / (Hq / Hkv) (grouped-query attention).
 * Dtypes.  ATTN_F32: float32 storage and float32 arithmetic throughout.
 *   ATTN_BF16: bfloat16 storage, bf16 matrix-core products with float32
 *   accumulation and float32 softmax statistics.  O, dQ, dK, dV take the
 *   input dtype (bf16 results rounded to nearest even); LSE is float32.
 * Mask.  causal != 0 allows key j for query i iff j <= i + (Skv - Sq)
 *   (bottom-right alignment; the usual lower triangle when Sq == Skv).  The
 *   definition requires every query row to keep at least one allowed key,
 *   so causal with Sq > Skv is rejected.
 * LSE.  lse[i] = m_i + ln(l_i): natural-log log-sum-exp of the scaled,
 *   masked scores of row i ("Don't Write Kernels, Derive Them", "What
 *   happened": logsumexp).
 * Scale.  Multiplies the exact dot product; must be finite.
 * Alignment.  Every pointer must be 16-byte aligned (128-bit accesses).
 * Aliasing.  No output may overlap an input or another output.
 * Stream.  `stream` is a hipStream_t (NULL = default stream).  Work is
 *   enqueued on it; results are valid once the stream passes the call.
 * Errors.  Arguments are checked on the host before anything is enqueued;
 *   on any error nothing is launched and a nonzero attn_status is returned.
 *   ATTN_ERR_HIP reports a failed launch (hipGetLastError) and then the
 *   state of the outputs is undefined.
 * Numerics.  Forward and decode are deterministic for fixed shapes and
 *   n_splits.  The backward writes each gradient element once (no atomics)
 *   and is deterministic too.  Inputs must be finite.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                       */
  ATTN_ERR_SHAPE = 2,       /* non-positive size, Hq % Hkv != 0, causal Sq>Skv,
                               sizes beyond the 32-bit per-head index range     */
  ATTN_ERR_UNSUPPORTED = 3, /* head dim or dtype outside the compiled set       */
  ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                 */
  ATTN_ERR_ALIAS = 5,       /* an output overlaps an input or another output    */
  ATTN_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than required          */
  ATTN_ERR_HIP = 7,         /* a HIP launch failed                              */
  ATTN_ERR_VALUE = 8        /* a scalar argument is invalid (scale not finite,
                               n_splits out of range, window without causal,
                               page size not a multiple of 32)                  */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Version of this ABI; bumped on any incompatible change. */
int attn_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* attn_status_str(int status);

/* Head dims compiled for (dtype, entry point): returns 1 if supported.
 * entry: 0 = attn_fwd, 1 = attn_decode, 2 = attn_bwd, 3 = attn_decode_paged,
 * 4 = attn_bwd_fused. */
int attn_supports(int dtype, int entry, int d);

/*
 * Forward prefill.  For every (b, h, i): O[b,h,i,:] and lse[b,h,i] of the
 * attention of query row i over the allowed keys of K/V head h / (Hq/Hkv).
 *   q   [B, Hq,  Sq,  d]   input
 *   k   [B, Hkv, Skv, d]   input
 *   v   [B, Hkv, Skv, d]   input
 *   o   [B, Hq,  Sq,  d]   output, dtype of the inputs
 *   lse [B, Hq,  Sq]       output, float32 (may be NULL if not wanted)
 * Computed as the blockwise recurrence of the second display equation of
 * "Compilers and Kernels", FlashAttention section, one query tile per
 * workgroup.  Supported d: f32 {64, 128, 256}; bf16 {64, 128, 256}.
 * Mask (the additive C of that section's first display equation):
 *   causal != 0: key j allowed for query i iff j <= i + (Skv - Sq);
 *   window > 0 (causal only, else ATTN_ERR_VALUE): also j > i + (Skv - Sq)
 *   - window, a sliding window of `window` keys ending at the diagonal;
 *   window <= 0: no window; window >= Skv masks no key the causal mask
 *   allows and runs as the plain causal call (the same kernels and bits);
 *   bias (may be NULL): float32 values added to the scaled scores,
 *   bias[b * bias_sb + h * bias_sh + i * Skv + j] for query head h (strides
 *   in elements, 0 to broadcast over batch or heads), any real or -inf; the
 *   pointer 16-byte aligned and Skv, bias_sb, bias_sh multiples of 4 (else
 *   ATTN_ERR_ALIGN), strides >= 0 (else ATTN_ERR_VALUE).  A row whose every
 *   key is masked gets O = 0 and lse = -inf.
 */
attn_status attn_fwd(int dtype, const void* q, const void* k, const void* v,
                     void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d,
                     int causal, int window, const float* bias, int64_t bias_sb,
                     int64_t bias_sh, float scale, void* stream);

/* Workspace for attn_decode: n_splits * B * Hq * (d + 2) float32 values,
 * rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int Hq, int d, int n_splits);

/*
 * Split-KV decode: one new query token per (batch, query head) against a
 * contiguous KV cache whose Skv keys are all visible (the cache already
 * holds the current token; no mask).
 *   q        [B, Hq, 1, d]     input
 *   k_cache  [B, Hkv, Skv, d]  input
 *   v_cache  [B, Hkv, Skv, d]  input
 *   o        [B, Hq, 1, d]     output, dtype of the inputs
 *   lse      [B, Hq, 1]        output, float32 (may be NULL)
 *   workspace >= attn_decode_workspace_bytes(B, Hq, d, n_splits) bytes of
 *             device memory, 16-byte aligned; contents on entry are ignored
 *             and on exit unspecified.
 * The keys are partitioned into n_splits sets: for bf16 with d in {64, 128},
 * split s takes the 32-key tiles s, s + n_splits, s + 2 n_splits, ...;
 * otherwise split s is the contiguous chunk [s c, (s + 1) c) with
 * c = ceil(Skv / n_splits).  Trailing splits may be empty.  A first kernel
 * computes each split's unnormalised state (m, l, acc) for all Hq / Hkv
 * query heads of a key/value head in one pass over that split's keys and
 * values; a second kernel folds the n_splits states of each query with the
 * monoid merge and writes O = acc / l and lse = m + ln l.  The state
 * (m, l, acc) is the one the blockwise recurrence of "Compilers and
 * Kernels" (section "FlashAttention changes the algorithm around IO", second
 * display equation) carries, and the merge is the monoid operation that
 * "Tang, a compiler that derives GPU kernels and bounds how fast they can
 * run" (Abstract) recognises online softmax as: both states rescaled to the
 * larger maximum and added.  It is associative and commutative, so every
 * partition gives the same result up to rounding.  1 <= n_splits <= 256,
 * else ATTN_ERR_VALUE.
 * Supported d: {64, 128, 256} for both dtypes.
 */
attn_status attn_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                        void* o, float* lse,
                        int B, int Hq, int Hkv, int Skv, int d, float scale, int n_splits,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged, variable-length split-KV decode: attn_decode over caches kept in
 * fixed-size pages of a shared pool and found through a block table
 * ("Don't Write Kernels, Derive Them", section "What happened": paged
 * KV-cache access is among the operations that emerge from the same
 * comprehensions); the result is attention of each stream's query over that
 * stream's keys in order.
 *   q           [B, Hq, 1, d]                         input
 *   k_pages     [n_pages, Hkv, page_size, d]          input, key pool
 *   v_pages     [n_pages, Hkv, page_size, d]          input, value pool
 *   block_table [B, max_pages] int32, device memory   input: key t of stream b
 *               is row t % page_size of page block_table[b][t / page_size]
 *   seq_lens    [B] int32, device memory              input: keys per stream,
 *               clamped to [0, max_pages * page_size]
 *   o           [B, Hq, 1, d]                         output, dtype of q
 *   lse         [B, Hq, 1] float32 (may be NULL)      output
 *   workspace   >= attn_decode_workspace_bytes(B, Hq, d, n_splits) bytes,
 *               16-byte aligned; contents on entry ignored, on exit unspecified.
 * The table and the lengths are read by the kernels, never by the host: a
 * page id outside [0, n_pages) reads as a page of zero keys and values (no
 * memory outside the pools is touched), and a stream with no keys gets
 * O = 0 and lse = -inf.  Split s of a stream takes its 32-key tiles s,
 * s + n_splits, ...; the splits are merged as in attn_decode.
 * bf16 only, d in {64, 128} (else ATTN_ERR_UNSUPPORTED); page_size a
 * multiple of 32 (else ATTN_ERR_VALUE); max_pages * page_size < 2^31 (else
 * ATTN_ERR_SHAPE); block_table and seq_lens 4-byte aligned, the other
 * pointers 16-byte aligned; 1 <= n_splits <= 256.  Two kernels, as
 * attn_decode.
 */
attn_status attn_decode_paged(int dtype, const void* q, const void* k_pages, const void* v_pages,
                              const int* block_table, const int* seq_lens, void* o, float* lse,
                              int B, int Hq, int Hkv, int d, int n_pages, int page_size,
                              int max_pages, float scale, int n_splits, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of the static device scratch that attn_decode_noalloc uses in place
 * of a workspace (8 MiB per device, held until the process ends). */
#define ATTN_SCRATCH_BYTES (8u << 20)

/*
 * attn_decode without a workspace, for callers that cannot allocate device
 * memory (code under graph capture, tight serving loops, harnesses that
 * forbid allocation): the same kernels, with the split states kept in a
 * static device array of ATTN_SCRATCH_BYTES bytes inside the library (one
 * per device, reserved for the life of the process) instead of a caller's
 * workspace.  The call allocates and frees nothing.
 *   Arguments, layouts, results and errors as attn_decode, without
 *   workspace and workspace_bytes; a problem whose states need more than
 *   ATTN_SCRATCH_BYTES, i.e. attn_decode_workspace_bytes(B, Hq, d, n_splits)
 *   > ATTN_SCRATCH_BYTES, returns ATTN_ERR_WORKSPACE with nothing launched.
 *   The first call on a device looks up that device's copy of the array
 *   (ATTN_ERR_HIP if that fails).
 * Every call on one device uses that device's one array: calls that overlap
 * on a device (other streams, other host threads) race on it and give
 * undefined results; serialise them.  Nothing in the array has to start at
 * any value (every split state is written before it is read), and it keeps
 * the last call's states.
 */
attn_status attn_decode_noalloc(int dtype, const void* q, const void* k_cache,
                                const void* v_cache, void* o, float* lse,
                                int B, int Hq, int Hkv, int Skv, int d, float scale,
                                int n_splits, void* stream);

/* Workspace for attn_bwd: 2 * B * Hq * Sqp float32 values, Sqp = Sq rounded
 * up to a multiple of 32 (per query row D_i = dO_i . O_i and
 * -lse_i * log2(e), with rows past Sq padded), rounded up to 256 bytes.
 * Returns 0 for invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Sq, int d);

/* The larger workspace that lets attn_bwd split the query heads of each
 * key/value head over several dK/dV workgroups per key tile (calls without
 * window and bias, on grids too small to fill the device: grouped heads,
 * few key/value heads): the pairs above, rounded up to 256 bytes, then p x 2
 * x B x Hkv x Skv x d float32 partial sums of dK and dV, for the split p
 * the library picks for this shape on the current device, or the one that
 * attn_bwd_tile_override forces on the calling thread (the plain size when
 * there is none).  attn_bwd takes the largest split its estimate
 * prefers that fits the workspace it is given.  Needs a current HIP device
 * (compute-unit count); returns 0 for invalid sizes. */
size_t attn_bwd_split_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int d,
                                      int causal);

/*
 * Backward.  Gradients of O = softmax(scale Q K^T + C) V given dO, with the
 * probabilities recomputed from the saved lse instead of being stored
 * ("Compilers and Kernels", FlashAttention section, closing paragraph; the
 * "Tang" Abstract: gradients of comprehensions are comprehensions):
 *   P = exp(scale Q K^T + C - lse), dV = P^T dO, dP = dO V^T,
 *   D_i = dO_i . O_i, dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q;
 * for grouped heads dK, dV of a key/value head sum over its query heads.
 *   q, k, v, o, d_o   inputs (o and lse as returned by attn_fwd)
 *   lse [B, Hq, Sq]   float32 input
 *   dq  [B, Hq, Sq, d], dk, dv [B, Hkv, Skv, d]   outputs, input dtype
 *   workspace >= attn_bwd_workspace_bytes(...) bytes, 16-byte aligned; that
 *   size must stay below 4 GiB (else ATTN_ERR_SHAPE).  A workspace of
 *   attn_bwd_split_workspace_bytes(...) bytes allows the head split (then a
 *   third kernel adds the partials into dk and dv).
 * causal, window and bias as in attn_fwd (the same mask as the forward
 * call; no gradient is formed for the bias).  Rows with lse = -inf (no
 * allowed key) contribute nothing.
 * Supported: bf16 with d in {64, 128, 256} (d = 256 at one wave per SIMD).
 */
attn_status attn_bwd(int dtype, const void* q, const void* k, const void* v,
                     const void* o, const void* d_o, const float* lse,
                     void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Skv, int d,
                     int causal, int window, const float* bias, int64_t bias_sb,
                     int64_t bias_sh, float scale,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for attn_bwd_fused: the attn_bwd workspace rounded up to 256
 * bytes, then B * Hq * Sq * d float32 values (the dQ accumulator), the total
 * rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t attn_bwd_fused_workspace_bytes(int B, int Hq, int Sq, int d);

/*
 * Fused backward: the gradients of attn_bwd (same formulas and arguments,
 * window and bias included) from one pass over the key tiles: the fused
 * kernel form of the backward that "Tang, a compiler that derives GPU
 * kernels and bounds how fast they can run" reports for CUDA in its Abstract
 * (a flash-style backward with no intermediates written, computing in bf16
 * and therefore outside an f32 tolerance).  Each workgroup owns 128 keys, forms dK and
 * dV for them while it loops over the query tiles, and adds its share
 * scale dS K of every query tile's dQ to a float32 accumulator in the
 * workspace with atomic adds; a last kernel rounds the accumulator to dq.
 * Three kernels per call: the (D, -lse log2 e) pairs with the accumulator
 * cleared, the fused dK/dV/dQ kernel, the dQ rounding.
 * Because the additions into the accumulator happen in no fixed order, dq
 * may differ in its last bits from call to call (dk and dv do not).
 *   workspace >= attn_bwd_fused_workspace_bytes(B, Hq, Sq, d) bytes,
 *   16-byte aligned; contents on entry are ignored, on exit unspecified.
 * Errors as attn_bwd.  Supported: bf16 with d in {64, 128}.
 */
attn_status attn_bwd_fused(int dtype, const void* q, const void* k, const void* v,
                           const void* o, const void* d_o, const float* lse,
                           void* dq, void* dk, void* dv,
                           int B, int Hq, int Hkv, int Sq, int Skv, int d,
                           int causal, int window, const float* bias, int64_t bias_sb,
                           int64_t bias_sh, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tile selection of the bf16 forward ("Tang, a compiler that derives GPU
 * kernels and bounds how fast they can run", Abstract: a per-tile traffic
 * and time estimate picks the tile).  Calls without a window or bias choose,
 * per shape, among compiled candidates (nw, bc, split): nw waves per
 * workgroup in `split` key groups of nw / split waves each, 32 nw / split
 * query rows per workgroup; key group g takes the bc-key tiles g,
 * g + split, g + 2 split, ... with its own softmax state, and the groups'
 * states of every row are merged at the end by the online-softmax monoid
 * (the same page, Abstract).  d64: (4,64,1) (4,32,1) (8,64,1) (2,64,1)
 * (4,32,4) (2,32,2) (4,64,2); d128: (4,32,1) (4,64,1) (8,32,1) (8,64,1)
 * (4,32,4) (2,32,2) (4,32,2); d256: (8,32,1) (4,32,1).  split = nw (one
 * 32-row block, every wave its own tiles) applies only where the grid has
 * at most one 32-row query block per compute unit.  Each candidate's time
 * is estimated from its per-tile matrix-core,
 * vector and synchronisation cycles, its occupancy on the device and a list
 * schedule of its workgroups; the fastest estimate wins, and the choice is
 * cached per (device, d, causal, B, Hq, Hkv, Sq, Skv).
 *
 * attn_fwd_tile_plan: the candidates for head dim d and the shape, up to cap
 *   of them written to nw[i], bc[i], split[i] and est_us[i] (estimated microseconds,
 *   +infinity for a candidate that does not apply to the shape; any array
 *   may be NULL), the index of the one a call would take to *pick.  Returns
 *   the number of candidates, 0 for an unsupported d or an invalid shape.
 *   Needs a current HIP device (occupancy query).
 * attn_fwd_tile_override: for the calling host thread, force (nw, bc, split)
 *   on later bf16 attn_fwd calls without window or bias (for sweeps and
 *   tests), whether or not the estimate would apply it; (0, 0, 0) returns to
 *   the estimate.  ATTN_ERR_VALUE unless all three are 0 or all positive
 *   with split dividing nw; a triple not compiled for a later call's d makes
 *   that call return ATTN_ERR_UNSUPPORTED.
 */
int attn_fwd_tile_plan(int d, int causal, int B, int Hq, int Hkv, int Sq, int Skv, int cap,
                       int* nw, int* bc, int* split, float* est_us, int* pick);
attn_status attn_fwd_tile_override(int nw, int bc, int split);

/*
 * attn_bwd_tile_override: for the calling host thread, force the launch
 * shapes of the two backward kernels on later attn_bwd calls (for sweeps
 * and tests).  dK/dV: nkw 32-key blocks per workgroup and hs groups of nkw
 * waves, each group taking every hs-th (query head, query tile) iteration;
 * dQ: nqw 32-row query blocks per workgroup and qhs groups of nqw waves,
 * each group taking every qhs-th key tile.  The groups' sums are added in
 * LDS at the end.  Each pair is (4, 1) (the plain kernel), (4, 2) or
 * (2, 4) (eight waves, the shapes the library takes on grids too small to
 * fill the compute units), or (0, 0) for the library's choice; d = 256
 * always runs (4, 1).  hsplit: the head split of the dK/dV kernel, 1 to 8
 * workgroups per key tile (0 = the library's choice; calls with window or
 * bias never split; a call whose workspace cannot hold the forced split
 * returns ATTN_ERR_WORKSPACE).  ATTN_ERR_VALUE for any other value.
 */
attn_status attn_bwd_tile_override(int nkw, int hs, int nqw, int qhs, int hsplit);

/*
 * attn_bwd_plan: the launch attn_bwd would make for a call of this shape on
 * the current device from the calling thread (its tile override included),
 * without launching anything: the dK/dV kernel's (nkw, hs), the dQ kernel's
 * (nqw, qhs), as in attn_bwd_tile_override, and the head split hsplit (1 =
 * none, then two kernels; else a third adds the partials).  window as in
 * attn_bwd; has_bias != 0 for a call that passes a bias (only its presence
 * matters); workspace_bytes the size of the workspace the call would get:
 * attn_bwd_workspace_bytes(...) never splits, attn_bwd_split_workspace_bytes
 * (...) allows the split the library prefers.  Status as attn_bwd would
 * return it for the sizes (ATTN_ERR_SHAPE, ATTN_ERR_VALUE,
 * ATTN_ERR_UNSUPPORTED for a head dim without a backward, ATTN_ERR_WORKSPACE
 * for a workspace below the plain size or one that cannot hold a forced
 * split), ATTN_ERR_NULL for a NULL output.  Without a HIP device the
 * estimate assumes 256 compute units.
 */
attn_status attn_bwd_plan(int B, int Hq, int Hkv, int Sq, int Skv, int d, int causal, int window,
                          int has_bias, size_t workspace_bytes, int* nkw, int* hs, int* nqw,
                          int* qhs, int* hsplit);

/*
 * Diagnostics: per-kernel timing.  `events` points to n hipEvent_t handles
 * created by the caller.  While set (per calling host thread), every entry
 * point binds events[2i] and events[2i+1] (those with index < n) to the i-th
 * kernel it launches, through hipExtLaunchKernel: they record that kernel's
 * start and end on its stream, with no packet of their own between kernels;
 * the caller reads the intervals with hipEventElapsedTime.  Kernels per call: attn_fwd 1
 * (the forward kernel), attn_decode and attn_decode_paged 2 (split,
 * combine), attn_bwd 2
 * (dQ together with D = rowsum(dO*O), then dK/dV; 3 with the head split:
 * then the partials' sum), attn_bwd_fused 3.  Pass NULL or n = 0 to stop.  The library
 * neither creates nor destroys the events.  Returns ATTN_ERR_VALUE if n < 0.
 */
attn_status attn_set_timing_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
