"""Seeded sweep of the backward's launch space against the float64 oracle:
random head dims, grouping, ragged and tiny lengths (Sq, Skv from 1),
causal / full, sliding window and additive bias, with the dK/dV and dQ
wave-group shapes and the head split either forced (attn_bwd_tile_override;
attn_bwd_plan must report what was forced) or left to the library (with the
workspace the binding allocates).  Cases are drawn once from a fixed seed,
so the list is the same on every run."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import randn, to_f64
from tests.gpu_util import TOL_GRAD, assert_close, inputs, note

pytestmark = pytest.mark.gpu

SHAPES = [(4, 1), (4, 2), (2, 4)]


def _cases(n=40, seed=20261203):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rs.choice([64, 128, 256], p=[0.35, 0.45, 0.2]))
        B = int(rs.choice([1, 2]))
        Hkv = int(rs.choice([1, 2, 3]))
        G = int(rs.choice([1, 2, 3, 4, 8]))
        causal = bool(rs.rand() < 0.7)
        mask = str(rs.choice(["none", "window", "bias"], p=[0.6, 0.2, 0.2]))
        if mask == "window" and not causal:
            mask = "none"
        Skv = int(rs.randint(1, 321))
        if mask == "bias":
            Skv = (Skv + 3) // 4 * 4   # the bias rows must stay 16-byte aligned
        Sq = int(rs.randint(1, Skv + 1)) if causal else int(rs.randint(1, 321))
        window = int(rs.randint(1, Skv + 11)) if mask == "window" else 0
        if rs.rand() < 0.4:
            launch = None   # the library's choice
        else:
            launch = (SHAPES[rs.randint(3)], SHAPES[rs.randint(3)], int(rs.choice([1, 2, 3, 4, 8])))
        out.append((i, B, Hkv * G, Hkv, Sq, Skv, d, causal, mask, window, launch))
    return out


# Edges the draw may miss: one query row, one key, a window at d256.
CASES = _cases() + [
    (40, 1, 8, 1, 1, 1, 128, True, "none", 0, ((2, 4), (2, 4), 8)),
    (41, 2, 4, 2, 1, 300, 64, True, "none", 0, None),
    (42, 1, 6, 3, 5, 1, 128, False, "none", 0, ((4, 2), (4, 1), 2)),
    (43, 1, 4, 2, 150, 200, 256, True, "window", 37, ((4, 1), (4, 1), 2)),
    (44, 2, 16, 2, 33, 33, 256, True, "none", 0, None),
]


def _id(c):
    i, B, Hq, Hkv, Sq, Skv, d, causal, mask, window, launch = c
    ln = "lib" if launch is None else "kv{}{}_q{}{}_p{}".format(*launch[0], *launch[1], launch[2])
    return (f"{i}_B{B}_Hq{Hq}_Hkv{Hkv}_Sq{Sq}_Skv{Skv}_d{d}_{'c' if causal else 'f'}_"
            f"{mask}{window or ''}_{ln}")


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_bwd_sweep(case):
    i, B, Hq, Hkv, Sq, Skv, d, causal, mask, window, launch = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 7000 + i, with_do=True)
    scale = 1 / math.sqrt(d)
    bias = None
    bias_ref = None
    if mask == "bias":
        bias = randn((B, Hq, Sq, Skv), 7500 + i, 0.5, torch.float32)
        bias_ref = bias.numpy().astype(np.float64)
        bias = bias.cuda()
    note(f"bwd sweep {_id(case)}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale,
                          window=window, bias=bias)
    masked = window > 0 and window < Skv or bias is not None
    if launch is None:
        dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                  causal=causal, scale=scale, window=window, bias=bias)
    else:
        kv, qs, p = launch
        aos.attn_bwd_tile_override(*kv, *qs, p)
        try:
            plain = aos.attn_bwd_workspace_bytes(B, Hq, Sq, d)
            need = max(plain, aos.attn_bwd_split_workspace_bytes(B, Hq, Hkv, Sq, Skv, d, causal))
            plan = aos.attn_bwd_plan(B, Hq, Hkv, Sq, Skv, d, causal, window=window,
                                     bias=bias is not None, workspace_bytes=need)
            if d <= 128:
                assert plan["dkdv"] == kv and plan["dq"] == qs
            else:
                assert plan["dkdv"] == (4, 1) and plan["dq"] == (4, 1)
            assert plan["hsplit"] == (1 if masked else p)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            dq, dk, dv = aos.attn_bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                      causal=causal, scale=scale, window=window, bias=bias,
                                      workspace=ws)
            torch.cuda.synchronize()
        finally:
            aos.attn_bwd_tile_override(0, 0, 0, 0, 0)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale,
                                             window=window, bias=bias_ref)
    assert_close(to_f64(dq), rq, TOL_GRAD, "sweep dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "sweep dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "sweep dV")
