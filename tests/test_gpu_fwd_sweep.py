"""Seeded sweeps of the forward and the decode against the float64 oracle.
Forward: random head dims, grouping, ragged and one-row lengths, causal /
full, window and bias, fp32 and bf16, with the bf16 tile candidate either
forced (any candidate the tile plan lists as applying to the shape) or
left to the estimate.  Decode: random shapes and split counts (1 to 64,
more splits than key tiles included), fp32 and bf16.  Cases are drawn once
from fixed seeds."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import randn, to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu


def _fwd_cases(n=40, seed=20261204):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        dt = "f32" if rs.rand() < 0.2 else "bf16"
        d = int(rs.choice([64, 128, 256], p=[0.35, 0.45, 0.2]))
        B = int(rs.choice([1, 2, 3]))
        Hkv = int(rs.choice([1, 2, 4]))
        G = int(rs.choice([1, 2, 4, 8]))
        causal = bool(rs.rand() < 0.6)
        mask = str(rs.choice(["none", "window", "bias"], p=[0.6, 0.2, 0.2]))
        if mask == "window" and not causal:
            mask = "none"
        Skv = int(rs.randint(1, 600))
        if mask == "bias":
            Skv = (Skv + 3) // 4 * 4   # the bias rows must stay 16-byte aligned
        Sq = int(rs.randint(1, Skv + 1)) if causal else int(rs.randint(1, 600))
        window = int(rs.randint(1, Skv + 11)) if mask == "window" else 0
        forced = dt == "bf16" and mask == "none" and rs.rand() < 0.6
        out.append((i, dt, B, Hkv * G, Hkv, Sq, Skv, d, causal, mask, window,
                    int(rs.randint(1 << 30)) if forced else None))
    return out


FWD_CASES = _fwd_cases() + [
    (40, "bf16", 1, 8, 2, 1, 1, 128, True, "none", 0, None),
    (41, "bf16", 2, 16, 2, 1, 700, 256, True, "none", 0, None),
    (42, "f32", 1, 4, 4, 3, 1, 64, False, "none", 0, None),
    (43, "bf16", 1, 4, 1, 260, 300, 256, True, "window", 31, None),
]


def _fid(c):
    i, dt, B, Hq, Hkv, Sq, Skv, d, causal, mask, window, pick = c
    return (f"{i}_{dt}_B{B}_Hq{Hq}_Hkv{Hkv}_Sq{Sq}_Skv{Skv}_d{d}_{'c' if causal else 'f'}_"
            f"{mask}{window or ''}_{'forced' if pick is not None else 'est'}")


@pytest.mark.parametrize("case", FWD_CASES, ids=_fid)
def test_fwd_sweep(case):
    i, dt, B, Hq, Hkv, Sq, Skv, d, causal, mask, window, pick = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, dt, 8000 + i)
    scale = 1 / math.sqrt(d)
    bias = bias_ref = None
    if mask == "bias":
        bias = randn((B, Hq, Sq, Skv), 8500 + i, 0.5, torch.float32)
        bias_ref = bias.numpy().astype(np.float64)
        bias = bias.cuda()
    forced = None
    if pick is not None:
        _, cands = aos.attn_fwd_tile_plan(d, causal, B, Hq, Hkv, Sq, Skv)
        usable = [c for c in cands if c["est_us"] is not None]
        if usable:
            forced = usable[pick % len(usable)]
    note(f"fwd sweep {_fid(case)} forced={forced}")
    if forced is not None:
        aos.attn_fwd_tile_override(forced["nw"], forced["bc"], forced["split"])
    try:
        o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale,
                              window=window, bias=bias)
        torch.cuda.synchronize()
    finally:
        aos.attn_fwd_tile_override(0, 0)
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale, window=window,
                                bias=bias_ref)
    assert_close(to_f64(o), O, TOL_O[dt], "sweep O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[dt], "sweep LSE")


def _dec_cases(n=24, seed=20261205):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        dt = "f32" if rs.rand() < 0.3 else "bf16"
        d = int(rs.choice([64, 128, 256]))
        Hkv = int(rs.choice([1, 2, 8]))
        G = int(rs.choice([1, 2, 4, 8, 16]))
        out.append((i, dt, int(rs.choice([1, 2, 5])), Hkv * G, Hkv, int(rs.randint(1, 3000)), d,
                    int(rs.choice([1, 2, 3, 7, 16, 31, 64]))))
    return out


DEC_CASES = _dec_cases()


@pytest.mark.parametrize("case", DEC_CASES,
                         ids=lambda c: "{}_{}_B{}_Hq{}_Hkv{}_Skv{}_d{}_n{}".format(*c))
def test_decode_sweep(case):
    i, dt, B, Hq, Hkv, Skv, d, n = case
    dev, ref = inputs(B, Hq, Hkv, 1, Skv, d, dt, 9000 + i)
    scale = 1 / math.sqrt(d)
    note(f"decode sweep {case}")
    o, lse = aos.attn_decode(dev["q"], dev["k"], dev["v"], scale=scale, n_splits=n)
    torch.cuda.synchronize()
    O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], scale, n)
    assert_close(to_f64(o), O, TOL_O[dt], "decode sweep O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[dt], "decode sweep LSE")


def _paged_cases(n=16, seed=20261206):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rs.choice([64, 128]))
        B = int(rs.randint(1, 5))
        Hkv = int(rs.choice([1, 2, 8]))
        G = int(rs.choice([1, 2, 4, 16]))
        ps = int(rs.choice([32, 64, 128, 256]))
        mp = int(rs.randint(1, 13))
        lens = [int(rs.randint(-2, ps * mp + 50)) for _ in range(B)]
        out.append((i, B, Hkv * G, Hkv, d, ps, mp, lens, int(rs.choice([1, 3, 16, 40]))))
    return out


@pytest.mark.parametrize("case", _paged_cases(),
                         ids=lambda c: "{}_B{}_Hq{}_Hkv{}_d{}_ps{}_mp{}_n{}".format(*c[:7], c[8]))
def test_paged_decode_sweep(case):
    """Random pages, table sizes and lengths (empty, negative, past the
    table's capacity: clamped)."""
    from tests.test_gpu_decode_paged import check
    from attention_online_softmax_amd.inputs import make_paged
    i, B, Hq, Hkv, d, ps, mp, lens, n = case
    cpu = make_paged(B, Hq, Hkv, d, ps, mp, lens, seed=9500 + i)
    dev = {k: v.cuda() for k, v in cpu.items()}
    scale = 1 / math.sqrt(d)
    note(f"paged decode sweep {case}")
    o, lse = aos.attn_decode_paged(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                                   dev["seq_lens"], scale=scale, n_splits=n)
    torch.cuda.synchronize()
    check(o, lse, cpu, scale, f"paged sweep {i}")


def _fused_cases(n=12, seed=20261207):
    rs = np.random.RandomState(seed)
    out = []
    for i in range(n):
        d = int(rs.choice([64, 128]))
        Hkv = int(rs.choice([1, 2]))
        G = int(rs.choice([1, 2, 4]))
        causal = bool(rs.rand() < 0.6)
        mask = str(rs.choice(["none", "window", "bias"], p=[0.5, 0.25, 0.25]))
        if mask == "window" and not causal:
            mask = "none"
        Skv = int(rs.randint(1, 300))
        if mask == "bias":
            Skv = (Skv + 3) // 4 * 4
        Sq = int(rs.randint(1, Skv + 1)) if causal else int(rs.randint(1, 300))
        window = int(rs.randint(1, Skv + 11)) if mask == "window" else 0
        out.append((i, int(rs.choice([1, 2])), Hkv * G, Hkv, Sq, Skv, d, causal, mask, window))
    return out


@pytest.mark.parametrize("case", _fused_cases(),
                         ids=lambda c: "{}_B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_{}{}".format(
                             *c[:7], "c" if c[7] else "f", c[8], c[9] or ""))
def test_fused_bwd_sweep(case):
    """The fused backward (dQ by float32 atomics) on random shapes and masks."""
    from tests.gpu_util import TOL_GRAD
    i, B, Hq, Hkv, Sq, Skv, d, causal, mask, window = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 9700 + i, with_do=True)
    scale = 1 / math.sqrt(d)
    bias = bias_ref = None
    if mask == "bias":
        bias = randn((B, Hq, Sq, Skv), 9800 + i, 0.5, torch.float32)
        bias_ref = bias.numpy().astype(np.float64)
        bias = bias.cuda()
    note(f"fused bwd sweep {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale,
                          window=window, bias=bias)
    dq, dk, dv = aos.attn_bwd_fused(dev["q"], dev["k"], dev["v"], o, dev["do"], lse,
                                    causal=causal, scale=scale, window=window, bias=bias)
    torch.cuda.synchronize()
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale,
                                             window=window, bias=bias_ref)
    assert_close(to_f64(dq), rq, TOL_GRAD, "fused sweep dQ")
    assert_close(to_f64(dk), rk, TOL_GRAD, "fused sweep dK")
    assert_close(to_f64(dv), rv, TOL_GRAD, "fused sweep dV")
