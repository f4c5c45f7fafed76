"""The backward kernels' eight-wave launch shapes for small grids, (4, 2)
and (2, 4): dK/dV with 32-key blocks per workgroup and groups of waves that
split the query iterations, dQ with 32-row blocks per workgroup and groups
that split the key tiles, the groups' sums added in LDS.  Forced through
attn_bwd_tile_override and checked against the float64 oracle, beside the
plain (4, 1) shapes on the same inputs."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import to_f64
from tests.gpu_util import TOL_GRAD, assert_close, inputs, note
from tests.test_gpu_bias import make_bias

pytestmark = pytest.mark.gpu

# (dK/dV shape, dQ shape)
SHAPES = [((4, 1), (4, 1)), ((4, 2), (4, 2)), ((2, 4), (2, 4)), ((4, 2), (2, 4)),
          ((2, 4), (4, 2))]

# (B, Hq, Hkv, Sq, Skv, d, causal, window, bias kind or None)
CASES = [
    (1, 8, 1, 300, 300, 128, True, 0, None),     # grouped heads, ragged tiles
    (1, 16, 2, 256, 256, 64, True, 0, None),
    (2, 4, 4, 130, 200, 128, True, 0, None),     # Sq < Skv, causal
    (1, 4, 2, 97, 161, 128, False, 0, None),
    (1, 2, 2, 33, 700, 64, True, 0, None),       # fewer query iterations than groups per tile
    (1, 1, 1, 1, 1, 64, False, 0, None),         # one query, one key
    (1, 3, 1, 64, 64, 128, True, 0, None),       # three query heads over four groups
    (1, 4, 1, 150, 150, 128, True, 40, None),    # sliding window
    (1, 4, 2, 100, 160, 64, False, 0, "head1"),  # additive bias, a dead row
    (1, 4, 1, 96, 96, 128, True, 33, "shared"),
]


def ids(c):
    return "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_w{}_{}".format(
        *c[:6], "causal" if c[6] else "full", c[7], c[8] or "nobias")


@pytest.mark.parametrize("case", CASES, ids=ids)
def test_dkdv_shapes_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal, W, kind = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 1700 + sum(case[:6]), with_do=True)
    scale = 1 / math.sqrt(d)
    bias = make_bias(kind, B, Hq, Sq, Skv, 1800 + sum(case[:6])) if kind else None
    bg = bias.cuda() if kind else None
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale, window=W,
                          bias=bg)
    bf = (np.broadcast_to(bias.numpy().astype(np.float64), (B, Hq, Sq, Skv)) if kind else None)
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal,
                                             scale, window=W, bias=bf)
    got = {}
    try:
        for kv, qs in SHAPES:
            note(f"bwd shapes dK/dV {kv} dQ {qs} {case}")
            aos.attn_bwd_tile_override(*kv, *qs, 1)
            dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                      causal=causal, scale=scale, window=W, bias=bg)
            torch.cuda.synchronize()
            assert_close(to_f64(dq), rq, TOL_GRAD, f"{kv}/{qs} dQ")
            assert_close(to_f64(dk), rk, TOL_GRAD, f"{kv}/{qs} dK")
            assert_close(to_f64(dv), rv, TOL_GRAD, f"{kv}/{qs} dV")
            got[(kv, qs)] = (dq, dk, dv)
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0)
    # dK/dV read only the (D, -lse log2 e) pairs from the dQ kernel, which
    # every dQ shape forms alike: the same dK/dV shape gives the same bits.
    for kv, q1, q2 in (((4, 2), (4, 2), (2, 4)), ((2, 4), (2, 4), (4, 2))):
        assert torch.equal(got[(kv, q1)][1], got[(kv, q2)][1])
        assert torch.equal(got[(kv, q1)][2], got[(kv, q2)][2])
    # dQ likewise depends only on its own shape.
    assert torch.equal(got[((4, 2), (2, 4))][0], got[((2, 4), (2, 4))][0])


def test_bwd_shapes_guard_regions():
    """Nothing is written past dQ, dK and dV by the grouped shapes (ragged
    queries and keys)."""
    B, Hq, Hkv, Sq, Skv, d = 1, 8, 1, 200, 170, 128
    dev, _ = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 1900, with_do=True)
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=False)
    pad = 4096
    try:
        for kv, qs in SHAPES[1:]:
            note(f"bwd guard dK/dV {kv} dQ {qs}")
            aos.attn_bwd_tile_override(*kv, *qs, 1)
            bufs, views = [], []
            for shape in ((B, Hq, Sq, d), (B, Hkv, Skv, d), (B, Hkv, Skv, d)):
                n = shape[0] * shape[1] * shape[2] * shape[3]
                buf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
                bufs.append((buf, n))
                views.append(buf[pad:pad + n].view(*shape))
            aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=False,
                         dq=views[0], dk=views[1], dv=views[2])
            torch.cuda.synchronize()
            for buf, n in bufs:
                assert torch.all(buf[:pad] == 7.0) and torch.all(buf[pad + n:] == 7.0)
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0)
