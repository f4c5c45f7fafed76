"""Backward through the C ABI against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import WORKLOADS, make_workload, to_f64
from tests.gpu_util import TOL_GRAD, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, Skv, d, causal)
CASES = [
    (1, 2, 2, 256, 256, 128, True),
    (1, 4, 2, 200, 200, 128, True),
    (2, 2, 1, 130, 300, 64, True),
    (1, 2, 2, 97, 161, 128, False),
    (1, 1, 1, 1, 1, 64, False),
    (1, 8, 1, 64, 64, 64, True),
    (1, 2, 2, 33, 2000, 128, True),
    (1, 2, 2, 200, 200, 256, True),
    (1, 4, 2, 130, 300, 256, True),
    (1, 2, 2, 97, 161, 256, False),
    (1, 8, 1, 64, 64, 256, True),
]


def run_case(dev, causal, scale):
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                              scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_bwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 500 + sum(case[:6]), with_do=True)
    scale = 1 / math.sqrt(d)
    note(f"bwd {case}")
    dq, dk, dv = run_case(dev, causal, scale)
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
    assert_close(to_f64(dq), rq, TOL_GRAD, "dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "dV")


def test_bwd_workload_full():
    """Training shape B4 H16 S2048 d128 causal: every gradient element."""
    w = WORKLOADS["train_fwd_bwd"]
    cpu = make_workload(w)
    dev = {k: v.cuda() for k, v in cpu.items()}
    note("bwd workload train_fwd_bwd")
    dq, dk, dv = run_case(dev, w.causal, w.scale)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], w.causal,
                                             w.scale)
    assert_close(to_f64(dq), rq, TOL_GRAD, "train dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "train dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "train dV")


def test_bwd_integrity():
    B, Hq, Hkv, S, d = 1, 4, 2, 190, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 71, with_do=True)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    keep = {k: v.clone() for k, v in dev.items()}
    keep_o, keep_l = o.clone(), lse.clone()
    dq = torch.full_like(dev["q"], float("nan"))
    dk = torch.full_like(dev["k"], float("nan"))
    dv = torch.full_like(dev["v"], float("nan"))
    note("bwd integrity")
    aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    for k in dev:
        assert torch.equal(dev[k], keep[k]), f"input {k} mutated"
    assert torch.equal(o, keep_o) and torch.equal(lse, keep_l)
    dq2, dk2, dv2 = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    # every input influences some gradient
    for name in ("q", "k", "v", "do"):
        pert = {k: v.clone() for k, v in dev.items()}
        pert[name][0, 1, 150, 3] += 1.0
        r = aos.attn_bwd(pert["q"], pert["k"], pert["v"], o, pert["do"], lse, causal=True)
        torch.cuda.synchronize()
        assert any(not torch.equal(a, b) for a, b in zip(r, (dq, dk, dv))), name
    l2 = lse.clone()
    l2[0, 1, 150] += 0.5
    r = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], l2, causal=True)
    torch.cuda.synchronize()
    assert any(not torch.equal(a, b) for a, b in zip(r, (dq, dk, dv))), "lse"


def test_bwd_gradient_identities():
    """Sum over keys of dK is zero and sum of dV equals sum of dO per head
    (exact identities of the definition), within bf16 rounding."""
    B, Hq, Hkv, S, d = 1, 4, 4, 256, 64
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 81, with_do=True)
    dq, dk, dv = run_case(dev, True, 1 / math.sqrt(d))
    sdk = dk.float().sum(dim=2)
    sdv = dv.float().sum(dim=2)
    sdo = dev["do"].float().sum(dim=2)
    assert float(sdk.abs().max()) < 0.1
    assert float((sdv - sdo).abs().max()) < 0.5
