"""Fused backward (dQ through fp32 atomic adds) through the C ABI: parity
with the float64 oracle, agreement with the two-kernel backward, and how far
its run-to-run results differ."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import WORKLOADS, make_workload, to_f64
from tests.gpu_util import TOL_GRAD, assert_close, inputs, note

pytestmark = pytest.mark.gpu


def bwd_plain(*args, **kw):
    """attn_bwd with its dK/dV kernel held to the plain (4, 1) shape: the
    fused kernel is that shape with dQ folded in, so their dK and dV agree
    bit for bit (the grouped shapes a small grid may take add the groups'
    sums in another order)."""
    aos.attn_bwd_tile_override(4, 1, 0, 0, 1)
    try:
        return aos.attn_bwd(*args, **kw)
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0)

# (B, Hq, Hkv, Sq, Skv, d, causal): ragged query and key tiles, grouped heads,
# Sq < Skv and Sq > Skv, key tiles shorter than the 128 keys of a workgroup,
# one-row and one-key inputs.
CASES = [
    (1, 2, 2, 256, 256, 128, True),
    (2, 4, 2, 200, 200, 64, True),
    (1, 4, 1, 96, 160, 128, True),
    (2, 2, 2, 130, 70, 128, False),
    (1, 2, 1, 33, 300, 64, False),
    (1, 8, 2, 257, 257, 128, True),
    (1, 1, 1, 1, 1, 64, False),
    (1, 2, 2, 33, 2000, 128, True),
]


def fwd(dev, causal, scale):
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_bwd_fused_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 1700 + sum(case[:6]), with_do=True)
    scale = 1 / math.sqrt(d)
    note(f"fused bwd {case}")
    o, lse = fwd(dev, causal, scale)
    dq, dk, dv = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                    causal=causal, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
    assert_close(to_f64(dq), rq, TOL_GRAD, "fused dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "fused dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "fused dV")
    # dK and dV come from the same products in the same order as the
    # two-kernel backward: bit for bit equal.
    _, dk2, dv2 = bwd_plain(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                               scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


# (B, Hq, Hkv, Sq, Skv, d, causal, window, bias kind or None)
MASKED = [
    (1, 4, 2, 150, 150, 128, True, 40, None),
    (1, 2, 1, 130, 200, 64, True, 33, None),
    (1, 4, 2, 100, 160, 64, False, 0, "head1"),
    (1, 2, 2, 128, 128, 128, True, 0, "full"),
    (1, 4, 1, 96, 96, 128, True, 33, "shared"),
]


@pytest.mark.parametrize("case", MASKED, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_w{}_{}".format(
    *c[:6], "causal" if c[6] else "full", c[7], c[8] or "nobias"))
def test_bwd_fused_window_bias(case):
    """The fused backward with a sliding window and an additive bias (a dead
    row included) against the oracle; dK and dV bit for bit equal to the
    two-kernel backward's plain shape."""
    from tests.test_gpu_bias import make_bias
    B, Hq, Hkv, Sq, Skv, d, causal, W, kind = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 2100 + sum(case[:6]), with_do=True)
    scale = 1 / math.sqrt(d)
    bias = make_bias(kind, B, Hq, Sq, Skv, 2200 + sum(case[:6])) if kind else None
    bg = bias.cuda() if kind else None
    note(f"fused bwd masked {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=W,
                          bias=bg)
    dq, dk, dv = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                    causal=causal, scale=scale, window=W, bias=bg)
    _, dk2, dv2 = bwd_plain(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                            scale=scale, window=W, bias=bg)
    torch.cuda.synchronize()
    bf = (np.broadcast_to(bias.numpy().astype(np.float64), (B, Hq, Sq, Skv)) if kind else None)
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal,
                                             scale, window=W, bias=bf)
    assert_close(to_f64(dq), rq, TOL_GRAD, "fused masked dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "fused masked dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "fused masked dV")
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_bwd_fused_workload_full():
    """Training shape B4 H16 S2048 d128 causal: every gradient element against
    the oracle; dK, dV equal to the two-kernel backward's; dQ of two fused
    calls and of the two-kernel backward within bf16 rounding of each other."""
    w = WORKLOADS["train_fwd_bwd"]
    cpu = make_workload(w)
    dev = {k: v.cuda() for k, v in cpu.items()}
    note("fused bwd workload train_fwd_bwd")
    o, lse = fwd(dev, w.causal, w.scale)
    dq, dk, dv = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                    causal=w.causal, scale=w.scale)
    dq_b, dk_b, dv_b = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                          causal=w.causal, scale=w.scale)
    dq2, dk2, dv2 = bwd_plain(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                 causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    ref = {k: to_f64(v) for k, v in cpu.items()}
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], w.causal,
                                             w.scale)
    assert_close(to_f64(dq), rq, TOL_GRAD, "fused train dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "fused train dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "fused train dV")
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.equal(dk, dk_b) and torch.equal(dv, dv_b)
    # dQ: the fp32 sums are formed in another order (and, between fused
    # calls, in no fixed order), so after rounding to bf16 an element may
    # move by one bf16 step of its magnitude.
    scale_q = float(dq2.float().abs().max())
    for other, what in ((dq_b, "fused vs fused"), (dq2, "fused vs two-kernel")):
        diff = (dq.float() - other.float()).abs()
        frac = float((diff > 0).float().mean())
        note(f"dQ {what}: max |diff| {float(diff.max()):.3e} "
             f"({float(diff.max()) / scale_q:.2e} of max |dQ|), {frac:.2e} of elements differ")
        step = other.float().abs() * 2.0 ** -7 + 1e-30
        assert bool((diff <= 2 * step + 1e-6 * scale_q).all()), what


def test_bwd_fused_integrity():
    """Inputs untouched, outputs finite, and the workspace contents on entry
    do not matter (the accumulator is cleared by the call itself)."""
    B, Hq, Hkv, S, d = 1, 4, 2, 190, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 1771, with_do=True)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    keep = {k: v.clone() for k, v in dev.items()}
    keep_o, keep_l = o.clone(), lse.clone()
    need = aos.attn_bwd_fused_workspace_bytes(B, Hq, S, d)
    ws = torch.full((need // 4,), float("nan"), device="cuda", dtype=torch.float32)
    note("fused bwd integrity")
    dq, dk, dv = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                                    workspace=ws)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    for k in dev:
        assert torch.equal(dev[k], keep[k]), f"input {k} mutated"
    assert torch.equal(o, keep_o) and torch.equal(lse, keep_l)
    ref = bwd_plain(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk, ref[1]) and torch.equal(dv, ref[2])
    assert_close(to_f64(dq), to_f64(ref[0]), 2e-2, "fused vs two-kernel dQ")
