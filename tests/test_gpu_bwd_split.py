"""The head split of the dK/dV kernel: the query heads of a key/value head
dealt over several workgroups per key tile, each writing float32 partial
sums of dK and dV into the workspace, and a third kernel adding them.
Forced through attn_bwd_tile_override on grouped-head shapes (and on one
without grouping) at d = 64, 128 and 256, checked against the float64
oracle; the library's own choice with the split workspace; the error for a
forced split the workspace cannot hold."""
import math

import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import to_f64
from tests.gpu_util import TOL_GRAD, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, Skv, d, causal)
CASES = [
    (1, 8, 1, 300, 300, 128, True),
    (2, 8, 2, 200, 260, 64, True),      # Sq < Skv
    (1, 4, 2, 130, 97, 128, False),     # ragged key tiles
    (1, 6, 2, 160, 160, 64, True),      # three query heads over two, four, eight shares
    (1, 8, 1, 256, 256, 256, True),
    (1, 4, 1, 97, 161, 256, False),
    (1, 2, 2, 128, 128, 128, True),     # no grouped heads: shares past the heads stay empty
]
SPLITS = [2, 4, 8]


def ids(c):
    return "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}".format(*c[:6], "causal" if c[6] else "full")


def ws_for(B, Hq, Hkv, Sq, Skv, d, p):
    plain = aos.attn_bwd_workspace_bytes(B, Hq, Sq, d)
    pairs = (plain + 255) // 256 * 256
    return pairs + p * 2 * B * Hkv * Skv * d * 4


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_head_split_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 2300 + sum(case[:6]), with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal,
                                             scale)
    shapes = [(4, 1)] if d > 128 else [(4, 1), (4, 2), (2, 4)]
    try:
        for p in SPLITS:
            ws = torch.empty(ws_for(B, Hq, Hkv, Sq, Skv, d, p), dtype=torch.uint8, device="cuda")
            for kv in shapes:
                note(f"bwd head split {p} dK/dV {kv} {case}")
                aos.attn_bwd_tile_override(*kv, 0, 0, p)
                dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                          causal=causal, scale=scale, workspace=ws)
                torch.cuda.synchronize()
                assert_close(to_f64(dq), rq, TOL_GRAD, f"split {p} {kv} dQ")
                assert_close(to_f64(dk), rk, TOL_GRAD, f"split {p} {kv} dK")
                assert_close(to_f64(dv), rv, TOL_GRAD, f"split {p} {kv} dV")
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0, 0)


def test_head_split_library_choice():
    """Grouped heads on a small grid with the split workspace the library
    asks for: its own choice (which splits here) against the oracle, and the
    same call with the plain workspace (which cannot split) within bf16
    rounding of it."""
    B, Hq, Hkv, S, d = 1, 16, 2, 1024, 128
    dev, ref = inputs(B, Hq, Hkv, S, S, d, "bf16", 2400, with_do=True)
    scale = 1 / math.sqrt(d)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    big = aos.attn_bwd_split_workspace_bytes(B, Hq, Hkv, S, S, d, True)
    small = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    assert big > small   # the estimate splits this shape
    note("bwd head split, library choice")
    got = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, scale=scale,
                       workspace=torch.empty(big, dtype=torch.uint8, device="cuda"))
    plain = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                         scale=scale,
                         workspace=torch.empty(small, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], True, scale)
    for g, r, what in zip(got, (rq, rk, rv), ("dQ", "dK", "dV")):
        assert_close(to_f64(g), r, TOL_GRAD, f"library split {what}")
    for a, b, what in zip(got, plain, ("dQ", "dK", "dV")):
        assert_close(to_f64(a), to_f64(b), TOL_GRAD, f"split vs plain workspace {what}")


def test_head_split_needs_its_workspace():
    B, Hq, Hkv, S, d = 1, 8, 1, 256, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 2500, with_do=True)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ws = torch.empty(ws_for(B, Hq, Hkv, S, S, d, 4) - 256, dtype=torch.uint8, device="cuda")
    aos.attn_bwd_tile_override(0, 0, 0, 0, 4)
    try:
        with pytest.raises(aos.AttnError, match="ATTN_ERR_WORKSPACE"):
            aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                         workspace=ws)
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0, 0)


def test_launch_follows_the_plan():
    """attn_bwd_plan says whether a call splits; the call's third kernel (the
    partials' sum) runs exactly then.  Events bound to kernel slot 2 are
    recorded before the call: they are recorded again after the dK/dV
    kernel only if that kernel is launched."""
    B, Hq, Hkv, S, d = 1, 16, 2, 1024, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 2600, with_do=True)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    big = aos.attn_bwd_split_workspace_bytes(B, Hq, Hkv, S, S, d, True)
    small = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    for ws_bytes in (big, small):
        plan = aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=ws_bytes)
        assert (plan["hsplit"] > 1) == (ws_bytes == big)
        note(f"bwd launch vs plan {plan}")
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in evs:
            e.record()
        torch.cuda.synchronize()
        aos.attn_set_timing_events([e.cuda_event for e in evs])
        try:
            aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                         workspace=torch.empty(ws_bytes, dtype=torch.uint8, device="cuda"))
        finally:
            aos.attn_set_timing_events(None)
        torch.cuda.synchronize()
        # the dK/dV kernel (slot 1) ran after the dQ kernel (slot 0)
        assert evs[0].elapsed_time(evs[3]) > 0
        third_ran = evs[3].elapsed_time(evs[4]) >= 0 and evs[3].elapsed_time(evs[5]) > 0
        assert third_ran == (plan["hsplit"] > 1)
