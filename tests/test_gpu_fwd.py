"""Forward prefill through the C ABI against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import WORKLOADS, make_workload, to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Sq, Skv, d, causal, dtype): several tiles plus ragged tails,
# grouped heads, Sq < Skv (bottom-right causal), single rows and single keys.
CASES = [
    (1, 1, 1, 128, 128, 64, False, "f32"),
    (1, 2, 1, 200, 333, 128, True, "f32"),
    (2, 2, 2, 65, 65, 256, True, "f32"),
    (1, 1, 1, 1, 1, 64, False, "f32"),
    (1, 1, 1, 17, 300, 64, False, "f32"),
    (1, 2, 1, 300, 300, 64, True, "bf16"),
    (1, 4, 2, 257, 511, 128, True, "bf16"),
    (1, 2, 1, 130, 130, 256, True, "bf16"),
    (2, 2, 2, 1, 1, 64, False, "bf16"),
    (1, 1, 1, 63, 1000, 128, False, "bf16"),
    (1, 2, 2, 129, 129, 128, False, "bf16"),
    (1, 8, 1, 100, 4000, 128, True, "bf16"),
    (1, 2, 2, 1, 777, 256, True, "bf16"),
    (3, 3, 1, 33, 97, 64, True, "bf16"),
]


def run_fwd(dev, causal, scale):
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}_{}".format(
    *c[:6], "causal" if c[6] else "full", c[7]))
def test_fwd_parity(case):
    B, Hq, Hkv, Sq, Skv, d, causal, dt = case
    seed = 100 + sum(case[:6])
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, dt, seed)
    scale = 1 / math.sqrt(d)
    note(f"fwd {case}")
    o, lse = run_fwd(dev, causal, scale)
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    assert_close(to_f64(o), O, TOL_O[dt], "O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[dt], "LSE")


@pytest.mark.parametrize("key", ["fp32_small", "block_fwd", "train_fwd_bwd"])
def test_fwd_workload_full(key):
    """Whole-output parity at the workload's own size."""
    w = WORKLOADS[key]
    cpu = make_workload(w)
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"fwd workload {key}")
    o, lse = run_fwd(dev, w.causal, w.scale)
    O, L = oracle.attention_ref(to_f64(cpu["q"]), to_f64(cpu["k"]), to_f64(cpu["v"]),
                                w.causal, w.scale)
    assert_close(to_f64(o), O, TOL_O[w.dtype], f"{key} O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[w.dtype], f"{key} LSE")


def test_fwd_long_prefill_sampled_rows():
    """44k-token d=256 grouped-query prefill: every head, the first 64, the
    last 64 and 128 random rows against the oracle computed row by row."""
    w = WORKLOADS["long_prefill"]
    cpu = make_workload(w)
    dev = {k: v.cuda() for k, v in cpu.items()}
    note("fwd long_prefill full size")
    o, lse = run_fwd(dev, w.causal, w.scale)
    rng = np.random.default_rng(4242)
    mid = rng.choice(np.arange(64, w.Sq - 64), size=128, replace=False)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(w.Sq - 64, w.Sq), mid]))
    O, L = oracle.attention_ref(to_f64(cpu["q"]), to_f64(cpu["k"]), to_f64(cpu["v"]),
                                w.causal, w.scale, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    assert_close(to_f64(o[:, :, idx]), O, TOL_O["bf16"], "long_prefill O rows")
    assert_close(lse[:, :, idx].cpu().numpy(), L, TOL_LSE["bf16"], "long_prefill LSE rows")
    assert torch.isfinite(o).all().item()


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fwd_integrity(dt):
    """Complete writes (NaN sentinels), no input mutation, bitwise
    determinism, and every input influences the output."""
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 190, 190, 128
    dev, _ = inputs(B, Hq, Hkv, Sq, Skv, d, dt, 77)
    keep = {k: v.clone() for k, v in dev.items()}
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), device="cuda")
    note(f"fwd integrity {dt}")
    aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, o=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    for k in dev:
        assert torch.equal(dev[k], keep[k]), f"input {k} mutated"
    o2, lse2 = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "not deterministic"
    for name in ("q", "k", "v"):
        pert = {k: v.clone() for k, v in dev.items()}
        pert[name][1, 1, 5, 3] += 1.0
        o3, lse3 = aos.attn_fwd(pert["q"], pert["k"], pert["v"], causal=True)
        torch.cuda.synchronize()
        assert not torch.equal(o3, o), f"output does not depend on {name}"


def test_fwd_streams():
    """Two calls on two streams give the same results as on one."""
    dev, _ = inputs(1, 4, 4, 256, 256, 64, "bf16", 91)
    dev2, _ = inputs(1, 4, 4, 256, 256, 64, "bf16", 92)
    ref1 = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    ref2 = aos.attn_fwd(dev2["q"], dev2["k"], dev2["v"], causal=True)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        a = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    with torch.cuda.stream(s2):
        b = aos.attn_fwd(dev2["q"], dev2["k"], dev2["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], ref1[0]) and torch.equal(b[0], ref2[0])


def test_fwd_errors_raise():
    dev, _ = inputs(1, 3, 2, 8, 8, 64, "bf16", 5)
    with pytest.raises(aos.AttnError):
        aos.attn_fwd(dev["q"], dev["k"], dev["v"])
    dev, _ = inputs(1, 2, 2, 9, 8, 64, "bf16", 5)
    with pytest.raises(aos.AttnError):
        aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)


# fp32 grids of at least 256 workgroups of 256 threads run the 256-thread
# configuration of the fp32 kernel (32 columns per lane); smaller grids,
# as in CASES above, the one-wave configuration (8 columns per lane).
F32_LARGE = [
    (2, 64, 16, 200, 250, 64, True),    # 2 x 64 heads x 2 tiles of 128 rows
    (1, 40, 8, 400, 300, 128, False),   # 40 heads x 7 tiles of 64 rows
    (1, 8, 2, 1100, 1100, 256, True),   # 8 heads x 35 tiles of 32 rows
]


@pytest.mark.parametrize("case", F32_LARGE, ids=lambda c: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_d{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_fwd_f32_large_grid(case):
    B, Hq, Hkv, Sq, Skv, d, causal = case
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "f32", 300 + sum(case[:6]))
    scale = 1 / math.sqrt(d)
    note(f"fwd f32 large grid {case}")
    o, lse = run_fwd(dev, causal, scale)
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    assert_close(to_f64(o), O, TOL_O["f32"], "O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE["f32"], "LSE")


def test_fwd_f32_large_grid_window_bias():
    """The 256-thread fp32 configuration with a sliding window and a
    per-batch additive bias (rows with no allowed key included)."""
    from tests.test_gpu_bias import check_fwd, make_bias
    B, Hq, Hkv, Sq, Skv, d, W = 2, 64, 64, 130, 132, 64, 50
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "f32", 777)
    bias = make_bias("head1", B, Hq, Sq, Skv, 778)
    scale = 1 / math.sqrt(d)
    note("fwd f32 large grid window + bias")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=W,
                          bias=bias.cuda())
    torch.cuda.synchronize()
    bf = np.broadcast_to(bias.numpy().astype(np.float64), (B, Hq, Sq, Skv))
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, scale, window=W, bias=bf)
    check_fwd(o, lse, O, L, "f32", "f32 large grid window + bias")
