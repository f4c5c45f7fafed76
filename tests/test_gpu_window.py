"""Causal sliding-window attention (forward and backward) through the C ABI
against the float64 oracle."""
import math

import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import to_f64
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, Skv, d, window, dtype): windows not aligned to tiles,
# Sq < Skv, a window of one key (the diagonal), a window wider than the
# keys, grouped heads, and the eight-wave d256 kernel.
FWD_CASES = [
    (1, 4, 2, 300, 300, 128, 100, "bf16"),
    (2, 2, 1, 200, 500, 64, 64, "bf16"),
    (1, 8, 2, 600, 600, 256, 257, "bf16"),
    (1, 2, 2, 129, 129, 128, 1, "bf16"),
    (1, 2, 1, 100, 100, 64, 1000, "bf16"),
    (1, 2, 2, 150, 150, 64, 33, "f32"),
    (1, 1, 1, 90, 200, 128, 17, "f32"),
    (1, 2, 2, 70, 70, 256, 5, "f32"),
    (1, 2, 1, 1, 100, 128, 10, "bf16"),
    (1, 2, 2, 5, 300, 64, 7, "f32"),
]

# (B, Hq, Hkv, Sq, Skv, d, window)
BWD_CASES = [
    (1, 2, 2, 256, 256, 128, 70),
    (2, 4, 2, 200, 330, 64, 128),
    (1, 8, 1, 300, 300, 128, 1),
    (1, 2, 2, 160, 160, 128, 1000),
    (1, 2, 1, 97, 161, 64, 40),
    (1, 2, 1, 3, 200, 64, 16),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_w{}_{}".format(
    *c))
def test_window_fwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, W, dt = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, dt, 900 + sum(case[:7]))
    scale = 1 / math.sqrt(d)
    note(f"window fwd {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=W)
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, scale, window=W)
    assert_close(to_f64(o), O, TOL_O[dt], "window O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[dt], "window LSE")


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_w{}".format(
    *c))
def test_window_bwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, W = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 950 + sum(case), with_do=True)
    scale = 1 / math.sqrt(d)
    note(f"window bwd {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=W)
    dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                              scale=scale, window=W)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], True, scale,
                                             window=W)
    assert_close(to_f64(dq), rq, TOL_GRAD, "window dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "window dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "window dV")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_window_wider_than_keys_is_causal(d):
    """A window of at least Skv keys masks nothing more than the causal mask:
    the outputs equal the plain causal call bit for bit (with the dK/dV head
    split held off: a masked call never splits, and a split sums the query
    heads' shares in another order)."""
    B, Hq, Hkv, Sq, Skv = 1, 4, 2, 300, 420
    dev, _ = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 990 + d, with_do=True)
    note(f"window >= Skv vs causal d={d}")
    oc, lc = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ow, lw = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, window=Skv)
    torch.cuda.synchronize()
    assert torch.equal(oc, ow) and torch.equal(lc, lw)
    if d <= 128:
        aos.attn_bwd_tile_override(0, 0, 0, 0, 1)
        try:
            gc = aos.attn_bwd(dev["q"], dev["k"], dev["v"], oc, dev["do"], lc, causal=True)
            gw = aos.attn_bwd(dev["q"], dev["k"], dev["v"], oc, dev["do"], lc, causal=True,
                              window=Skv + 7)
            torch.cuda.synchronize()
        finally:
            aos.attn_bwd_tile_override(0, 0, 0, 0, 0)
        for a, b in zip(gc, gw):
            assert torch.equal(a, b)


def test_window_long():
    """S = 2048 with a 512-key window: many tiles fully inside, outside and
    cut by the window's lower edge."""
    B, Hq, Hkv, S, d, W = 1, 2, 1, 2048, 128, 512
    dev, ref = inputs(B, Hq, Hkv, S, S, d, "bf16", 997, with_do=True)
    scale = 1 / math.sqrt(d)
    note("window long S2048 W512")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=W)
    dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=True,
                              scale=scale, window=W)
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, scale, window=W)
    assert_close(to_f64(o), O, TOL_O["bf16"], "long window O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE["bf16"], "long window LSE")
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], True, scale,
                                             window=W)
    assert_close(to_f64(dq), rq, TOL_GRAD, "long window dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "long window dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "long window dV")
