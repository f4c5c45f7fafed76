"""Additive bias (the general mask C) through the C ABI against the float64
oracle, forward and backward."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import randn, to_f64
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu


def make_bias(kind, B, Hq, Sq, Skv, seed, dead_row=True):
    """fp32 bias of shape [B|1, Hq|1, Sq, Skv]: N(0, 2^2) values, about one
    entry in ten set to -inf, and (dead_row) one row masked entirely."""
    shape = {"full": (B, Hq), "batch1": (1, Hq), "head1": (B, 1), "shared": (1, 1)}[kind]
    t = randn(shape + (Sq, Skv), seed, 2.0, torch.float32)
    drop = randn(shape + (Sq, Skv), seed + 1, 1.0, torch.float32) > 1.3
    t[drop] = -math.inf
    if dead_row:
        t[0, 0, Sq // 2, :] = -math.inf
    return t


def check_fwd(o, lse, O, L, dt, what):
    got_o, got_l = to_f64(o), lse.cpu().numpy().astype(np.float64)
    dead = np.isinf(L)
    assert np.array_equal(np.isinf(got_l), dead), f"{what}: rows without keys differ"
    assert np.all(got_l[dead] < 0) and np.all(got_o[dead] == 0), f"{what}: empty rows"
    assert_close(got_o, O, TOL_O[dt], f"{what} O")
    assert_close(np.where(dead, 0, got_l), np.where(dead, 0, L), TOL_LSE[dt], f"{what} LSE")


# (B, Hq, Hkv, Sq, Skv, d, causal, window, bias kind, dtype)
FWD_CASES = [
    (2, 4, 2, 100, 140, 64, False, 0, "full", "bf16"),
    (1, 4, 2, 200, 200, 128, True, 0, "head1", "bf16"),
    (2, 2, 2, 64, 96, 128, False, 0, "shared", "bf16"),
    (1, 2, 2, 130, 132, 128, True, 40, "full", "bf16"),
    (1, 2, 1, 50, 52, 64, True, 0, "full", "f32"),
    (2, 2, 2, 33, 36, 256, False, 0, "batch1", "f32"),
    (1, 2, 1, 100, 128, 256, True, 0, "full", "bf16"),
    (2, 2, 2, 64, 96, 256, False, 0, "head1", "bf16"),
    (1, 2, 2, 130, 132, 256, True, 40, "shared", "bf16"),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_w{}_{}_{}".format(
    *c[:6], "causal" if c[6] else "full", *c[7:]))
def test_bias_fwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal, W, kind, dt = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, dt, 1100 + sum(case[:6]))
    bias = make_bias(kind, B, Hq, Sq, Skv, 1200 + sum(case[:6]))
    scale = 1 / math.sqrt(d)
    note(f"bias fwd {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=W,
                          bias=bias.cuda())
    torch.cuda.synchronize()
    bf = np.broadcast_to(bias.numpy().astype(np.float64), (B, Hq, Sq, Skv))
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale, window=W, bias=bf)
    check_fwd(o, lse, O, L, dt, f"bias {case}")


# (B, Hq, Hkv, Sq, Skv, d, causal, window, bias kind)
BWD_CASES = [
    (1, 2, 2, 128, 128, 128, True, 0, "full"),
    (2, 4, 2, 100, 160, 64, False, 0, "head1"),
    (1, 4, 1, 96, 96, 128, True, 33, "shared"),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_w{}_{}".format(
    *c[:6], "causal" if c[6] else "full", *c[7:]))
def test_bias_bwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal, W, kind = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 1300 + sum(case[:6]), with_do=True)
    bias = make_bias(kind, B, Hq, Sq, Skv, 1400 + sum(case[:6]))
    scale = 1 / math.sqrt(d)
    note(f"bias bwd {case}")
    bg = bias.cuda()
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=W,
                          bias=bg)
    dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                              scale=scale, window=W, bias=bg)
    torch.cuda.synchronize()
    bf = np.broadcast_to(bias.numpy().astype(np.float64), (B, Hq, Sq, Skv))
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale,
                                             window=W, bias=bf)
    assert_close(to_f64(dq), rq, TOL_GRAD, "bias dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "bias dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "bias dV")


def test_bias_causal_pattern_equals_causal():
    """The causal pattern written as a 0 / -inf bias gives the causal result."""
    B, Hq, Hkv, S, d = 1, 4, 2, 256, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 1500, with_do=True)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    bias = torch.where(j <= i, 0.0, -math.inf).to(torch.float32)[None, None].cuda()
    note("bias = causal pattern")
    oc, lc = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ob, lb = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=False, bias=bias)
    gc = aos.attn_bwd(dev["q"], dev["k"], dev["v"], oc, dev["do"], lc, causal=True)
    gb = aos.attn_bwd(dev["q"], dev["k"], dev["v"], ob, dev["do"], lb, causal=False, bias=bias)
    torch.cuda.synchronize()
    assert_close(to_f64(ob), to_f64(oc), 2e-2, "bias-causal O")
    assert_close(lb.cpu().numpy(), lc.cpu().numpy(), 1e-3, "bias-causal LSE")
    for a, b, nm in zip(gb, gc, ("dQ", "dK", "dV")):
        assert_close(to_f64(a), to_f64(b), 5e-2, f"bias-causal {nm}")
