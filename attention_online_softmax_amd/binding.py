"""ctypes binding over libattn.so: argument marshalling only.

Every function here checks that tensors are contiguous device tensors of one
dtype, allocates outputs and workspaces with torch when the caller does not
pass them, and calls the C entry point of the same name on torch's current
stream.  All arithmetic happens in the HIP kernels; there is no fallback: if
the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
STATUS_NAMES = {
    0: "ATTN_OK", 1: "ATTN_ERR_NULL", 2: "ATTN_ERR_SHAPE", 3: "ATTN_ERR_UNSUPPORTED",
    4: "ATTN_ERR_ALIGN", 5: "ATTN_ERR_ALIAS", 6: "ATTN_ERR_WORKSPACE", 7: "ATTN_ERR_HIP",
    8: "ATTN_ERR_VALUE",
}
EXPORTS = ("attn_abi_version", "attn_status_str", "attn_supports", "attn_fwd",
           "attn_decode_workspace_bytes", "attn_decode", "attn_decode_paged",
           "attn_bwd_workspace_bytes", "attn_bwd_split_workspace_bytes", "attn_bwd_plan",
           "attn_bwd",
           "attn_bwd_fused_workspace_bytes",
           "attn_bwd_fused", "attn_set_timing_events", "attn_decode_noalloc",
           "attn_fwd_tile_plan", "attn_fwd_tile_override", "attn_bwd_tile_override")
SCRATCH_BYTES = 8 << 20   # ATTN_SCRATCH_BYTES of attn.h

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({attn_status_str(status)})")


def lib():
    """Load libattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m attention_online_softmax_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_abi_version.restype = i
    L.attn_abi_version.argtypes = []
    L.attn_status_str.restype = ctypes.c_char_p
    L.attn_status_str.argtypes = [i]
    L.attn_supports.restype = i
    L.attn_supports.argtypes = [i, i, i]
    L.attn_fwd.restype = i
    i64 = ctypes.c_int64
    L.attn_fwd.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, i64, i64, f, vp]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_decode_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_decode.restype = i
    L.attn_decode.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    L.attn_decode_noalloc.restype = i
    L.attn_decode_noalloc.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.attn_decode_paged.restype = i
    L.attn_decode_paged.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp,
                                    sz, vp]
    L.attn_bwd_workspace_bytes.restype = sz
    L.attn_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_bwd.restype = i
    L.attn_bwd.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                           i, i, i, i, i, i, i, i, vp, i64, i64, f, vp, sz, vp]
    L.attn_bwd_fused_workspace_bytes.restype = sz
    L.attn_bwd_fused_workspace_bytes.argtypes = [i, i, i, i]
    L.attn_bwd_fused.restype = i
    L.attn_bwd_fused.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                 i, i, i, i, i, i, i, i, vp, i64, i64, f, vp, sz, vp]
    ip, fp = ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_float)
    L.attn_fwd_tile_plan.restype = i
    L.attn_fwd_tile_plan.argtypes = [i, i, i, i, i, i, i, i, ip, ip, ip, fp, ip]
    L.attn_fwd_tile_override.restype = i
    L.attn_fwd_tile_override.argtypes = [i, i, i]
    L.attn_bwd_tile_override.restype = i
    L.attn_bwd_tile_override.argtypes = [i, i, i, i, i]
    L.attn_bwd_split_workspace_bytes.restype = sz
    L.attn_bwd_split_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    L.attn_bwd_plan.restype = i
    L.attn_bwd_plan.argtypes = [i, i, i, i, i, i, i, i, i, sz] + [ctypes.POINTER(i)] * 5
    L.attn_set_timing_events.restype = i
    L.attn_set_timing_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), i]
    _lib = L
    return L


def attn_abi_version():
    return lib().attn_abi_version()


def attn_status_str(status):
    return lib().attn_status_str(int(status)).decode()


def attn_supports(dtype, entry, d):
    return bool(lib().attn_supports(int(dtype), int(entry), int(d)))


def attn_set_timing_events(events):
    """events: sequence of raw hipEvent_t handles (ints), or None to stop.
    Slot 2i is recorded before and 2i+1 after the i-th kernel of each call."""
    if not events:
        st = lib().attn_set_timing_events(None, 0)
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        attn_set_timing_events._keep = arr  # the library keeps the pointer
        st = lib().attn_set_timing_events(arr, len(events))
    if st:
        raise AttnError(st, "attn_set_timing_events")


def attn_fwd_tile_plan(d, causal, B, Hq, Hkv, Sq, Skv):
    """The bf16 forward's tile candidates for a shape: a list of
    {"nw", "bc", "split", "est_us"} and the index the estimate picks (None, []
    for an unsupported head dim or shape).  nw waves in `split` key groups,
    32 nw / split query rows per workgroup (split = nw: the key-split kernel
    on one 32-row block); est_us is None where a candidate does not apply
    to the shape."""
    cap = 16
    nw, bc, sp = (ctypes.c_int * cap)(), (ctypes.c_int * cap)(), (ctypes.c_int * cap)()
    est, pick = (ctypes.c_float * cap)(), ctypes.c_int(-1)
    n = lib().attn_fwd_tile_plan(int(d), int(bool(causal)), B, Hq, Hkv, Sq, Skv, cap, nw, bc, sp,
                                 est, ctypes.byref(pick))
    cands = [{"nw": nw[i], "bc": bc[i], "split": sp[i],
              "est_us": est[i] if math.isfinite(est[i]) else None} for i in range(min(n, cap))]
    return (pick.value if n else None), cands


def attn_fwd_tile_override(nw=0, bc=0, split=1):
    """Force (waves per workgroup, keys per tile, key groups) on this
    thread's later bf16 forward calls without window or bias; nw = bc = 0
    returns to the estimate."""
    if nw == 0 and bc == 0:
        split = 0
    st = lib().attn_fwd_tile_override(int(nw), int(bc), int(split))
    if st:
        raise AttnError(st, "attn_fwd_tile_override")


def attn_bwd_tile_override(nkw=0, hs=0, nqw=0, qhs=0, hsplit=0):
    """Force the launch shapes of the backward kernels on this thread's later
    calls: dK/dV (32-key blocks per workgroup, wave groups) and dQ (32-row
    blocks per workgroup, wave groups), each (4, 1), (4, 2) or (2, 4) at
    d <= 128, and the dK/dV head split (1 to 8 workgroups per key tile);
    zeros leave each to the library's choice."""
    st = lib().attn_bwd_tile_override(int(nkw), int(hs), int(nqw), int(qhs), int(hsplit))
    if st:
        raise AttnError(st, "attn_bwd_tile_override")


def attn_decode_workspace_bytes(B, Hq, d, n_splits):
    return int(lib().attn_decode_workspace_bytes(B, Hq, d, n_splits))


def attn_bwd_workspace_bytes(B, Hq, Sq, d):
    return int(lib().attn_bwd_workspace_bytes(B, Hq, Sq, d))


def _dtype_code(t):
    if t.dtype == torch.float32:
        return ATTN_F32
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(ts, names):
    dev = ts[0].device
    for t, nm in zip(ts, names):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{nm} must be a tensor")
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError(f"{nm} must be on the same GPU as {names[0]}")
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _bias_args(bias, B, Hq, Sq, Skv, dev):
    """(pointer, batch stride, head stride) of an additive fp32 bias that
    broadcasts to [B, Hq, Sq, Skv] (size-1 batch / head dimensions broadcast;
    the last two dimensions must be contiguous)."""
    if bias is None:
        return None, 0, 0
    if not isinstance(bias, torch.Tensor) or bias.dtype != torch.float32 or bias.device != dev:
        raise TypeError("bias must be a float32 tensor on the same GPU")
    if bias.dim() != 4 or tuple(bias.shape[2:]) != (Sq, Skv) or bias.shape[0] not in (1, B) \
            or bias.shape[1] not in (1, Hq):
        raise ValueError("bias must broadcast to [B, Hq, Sq, Skv]")
    if bias.stride(3) != 1 or bias.stride(2) != Skv:
        raise ValueError("bias rows must be contiguous [Sq, Skv] planes")
    sb = bias.stride(0) if bias.shape[0] == B and B > 1 else 0
    sh = bias.stride(1) if bias.shape[1] == Hq and Hq > 1 else 0
    return _ptr(bias), sb, sh


def attn_fwd(q, k, v, causal=False, scale=None, o=None, lse=None, stream=None, want_lse=True,
             window=0, bias=None):
    """Forward prefill.  q [B,Hq,Sq,d], k/v [B,Hkv,Skv,d]; returns (o, lse).
    window > 0 (with causal): a sliding window of that many keys.
    bias: optional fp32 additive mask broadcasting to [B, Hq, Sq, Skv]."""
    _check([q, k, v], ["q", "k", "v"])
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Sq), device=q.device, dtype=torch.float32)
    dt = _dtype_code(q)
    st = lib().attn_fwd(dt, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                        B, Hq, Hkv, Sq, Skv, d, int(bool(causal)), int(window),
                        *_bias_args(bias, B, Hq, Sq, Skv, q.device), float(scale),
                        _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_fwd")
    return o, lse


def attn_decode(q, k_cache, v_cache, scale=None, n_splits=16, o=None, lse=None,
                workspace=None, stream=None):
    """Split-KV decode.  q [B,Hq,1,d], caches [B,Hkv,Skv,d]; returns (o, lse)."""
    _check([q, k_cache, v_cache], ["q", "k_cache", "v_cache"])
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per head: q must be [B, Hq, 1, d]")
    Hkv, Skv = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, 1), device=q.device, dtype=torch.float32)
    need = attn_decode_workspace_bytes(B, Hq, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    st = lib().attn_decode(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                           _ptr(lse), B, Hq, Hkv, Skv, d, float(scale), int(n_splits),
                           _ptr(workspace), workspace.numel() * workspace.element_size(),
                           _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_decode")
    return o, lse


def attn_decode_noalloc(q, k_cache, v_cache, scale=None, n_splits=16, o=None, lse=None,
                        stream=None):
    """attn_decode with the split states in the library's static device
    scratch instead of a workspace (the library allocates nothing; outputs
    are allocated here only if not passed).  Calls that overlap on one GPU
    race on that scratch.  Returns (o, lse)."""
    _check([q, k_cache, v_cache], ["q", "k_cache", "v_cache"])
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per head: q must be [B, Hq, 1, d]")
    Hkv, Skv = k_cache.shape[1], k_cache.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, 1), device=q.device, dtype=torch.float32)
    st = lib().attn_decode_noalloc(_dtype_code(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o),
                                   _ptr(lse), B, Hq, Hkv, Skv, d, float(scale), int(n_splits),
                                   _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_decode_noalloc")
    return o, lse


def attn_decode_paged(q, k_pages, v_pages, block_table, seq_lens, scale=None, n_splits=16,
                      o=None, lse=None, workspace=None, stream=None):
    """Paged, variable-length decode.  q [B,Hq,1,d]; pools [n_pages,Hkv,page_size,d];
    block_table [B,max_pages] and seq_lens [B] int32 on the same GPU; returns (o, lse)."""
    _check([q, k_pages, v_pages, block_table, seq_lens],
           ["q", "k_pages", "v_pages", "block_table", "seq_lens"])
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per head: q must be [B, Hq, 1, d]")
    n_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if tuple(v_pages.shape) != tuple(k_pages.shape) or tuple(block_table.shape[:1]) != (B,) \
            or tuple(seq_lens.shape) != (B,):
        raise ValueError("inconsistent paged-cache shapes")
    max_pages = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, 1), device=q.device, dtype=torch.float32)
    need = attn_decode_workspace_bytes(B, Hq, d, n_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    st = lib().attn_decode_paged(_dtype_code(q), _ptr(q), _ptr(k_pages), _ptr(v_pages),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                 d, n_pages, page_size, max_pages, float(scale), int(n_splits),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_decode_paged")
    return o, lse


def attn_bwd(q, k, v, o, do, lse, causal=False, scale=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, window=0, bias=None):
    """Backward (same causal / window as the forward call).  Returns (dq, dk, dv).

    Without a `workspace`, one is allocated for the call: for calls without
    window and bias, the size of attn_bwd_split_workspace_bytes, which lets
    the library deal a key/value head's query heads over several workgroups
    (float32 partials of dK and dV, up to 8 x 2 x B x Hkv x Skv x d x 4
    bytes on grids too small to fill the device); else the pairs alone.  Pass
    a workspace of attn_bwd_workspace_bytes to keep the call within that."""
    _check([q, k, v, o, do, lse], ["q", "k", "v", "o", "do", "lse"])
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        # the size that lets the library split grouped heads when it wants to
        need = (attn_bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, causal)
                if window == 0 and bias is None else attn_bwd_workspace_bytes(B, Hq, Sq, d))
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    st = lib().attn_bwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                        _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Skv, d,
                        int(bool(causal)), int(window), *_bias_args(bias, B, Hq, Sq, Skv, q.device),
                        float(scale), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_bwd")
    return dq, dk, dv


def attn_bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, causal):
    return int(lib().attn_bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, int(bool(causal))))


def attn_bwd_plan(B, Hq, Hkv, Sq, Skv, d, causal, window=0, bias=False, workspace_bytes=None):
    """The launch attn_bwd would make: {"dkdv": (nkw, hs), "dq": (nqw, qhs),
    "hsplit": p}.  workspace_bytes defaults to the size attn_bwd allocates
    itself when given none (the split workspace for calls without window or
    bias).  Raises AttnError with the status attn_bwd would return."""
    if workspace_bytes is None:
        workspace_bytes = attn_bwd_workspace_bytes(B, Hq, Sq, d)
        if window <= 0 and not bias:
            workspace_bytes = max(workspace_bytes,
                                  attn_bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, causal))
    out = [ctypes.c_int() for _ in range(5)]
    st = lib().attn_bwd_plan(B, Hq, Hkv, Sq, Skv, d, int(bool(causal)), int(window),
                             int(bool(bias)), int(workspace_bytes), *[ctypes.byref(x) for x in out])
    if st != 0:
        raise AttnError(st, "attn_bwd_plan")
    v = [x.value for x in out]
    return {"dkdv": (v[0], v[1]), "dq": (v[2], v[3]), "hsplit": v[4]}


def attn_bwd_fused_workspace_bytes(B, Hq, Sq, d):
    return int(lib().attn_bwd_fused_workspace_bytes(B, Hq, Sq, d))


def attn_bwd_fused(q, k, v, o, do, lse, causal=False, scale=None, dq=None, dk=None, dv=None,
                   workspace=None, stream=None, window=0, bias=None):
    """Fused backward (dQ through fp32 atomic adds; window and bias as in
    attn_bwd).  Returns (dq, dk, dv)."""
    _check([q, k, v, o, do, lse], ["q", "k", "v", "o", "do", "lse"])
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_bwd_fused_workspace_bytes(B, Hq, Sq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 256), device=q.device, dtype=torch.uint8)
    st = lib().attn_bwd_fused(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do),
                              _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, Sq, Skv, d,
                              int(bool(causal)), int(window),
                              *_bias_args(bias, B, Hq, Sq, Skv, q.device), float(scale),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream, q.device))
    if st:
        raise AttnError(st, "attn_bwd_fused")
    return dq, dk, dv
