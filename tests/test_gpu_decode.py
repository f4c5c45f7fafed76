"""Split-KV decode through the C ABI against the float64 oracle."""
import math

import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import WORKLOADS, make_workload, to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Skv, d, n_splits, dtype): grouped heads from 1 to 16 per
# key/value head (16 uses two head chunks), ragged chunks, empty trailing
# chunks (n_splits * chunk > Skv), a single key, one split, and splits of
# more than 1024 keys on every kernel (bf16 d128 on the matrix cores, fp32
# and bf16 d256 on the vector units).
CASES = [
    (2, 8, 2, 1000, 128, 16, "bf16"),
    (1, 4, 4, 513, 64, 7, "bf16"),
    (1, 16, 1, 300, 256, 5, "bf16"),
    (2, 2, 1, 1, 128, 1, "bf16"),
    (1, 4, 1, 10, 128, 16, "bf16"),
    (1, 8, 1, 1024, 128, 1, "bf16"),
    (1, 8, 2, 3000, 128, 1, "bf16"),
    (1, 4, 2, 2100, 256, 1, "bf16"),
    (2, 4, 1, 2500, 64, 2, "f32"),
    (2, 8, 2, 777, 128, 16, "f32"),
    (1, 3, 1, 200, 64, 3, "f32"),
    (1, 2, 2, 90, 256, 4, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_Skv{}_d{}_n{}_{}".format(*c))
def test_decode_parity(case):
    B, Hq, Hkv, Skv, d, n, dt = case
    dev, ref = inputs(B, Hq, Hkv, 1, Skv, d, dt, 300 + sum(case[:6]))
    scale = 1 / math.sqrt(d)
    note(f"decode {case}")
    o, lse = aos.attn_decode(dev["q"], dev["k"], dev["v"], scale=scale, n_splits=n)
    torch.cuda.synchronize()
    O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], scale, n)
    assert_close(to_f64(o), O, TOL_O[dt], "decode O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE[dt], "decode LSE")


def test_decode_workload_full():
    w = WORKLOADS["gqa_decode"]
    cpu = make_workload(w)
    dev = {k: v.cuda() for k, v in cpu.items()}
    note("decode workload gqa_decode")
    o, lse = aos.attn_decode(dev["q"], dev["k"], dev["v"], scale=w.scale, n_splits=w.n_splits)
    torch.cuda.synchronize()
    ref = {k: to_f64(v) for k, v in cpu.items()}
    O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], w.scale, w.n_splits)
    assert_close(to_f64(o), O, TOL_O["bf16"], "gqa_decode O")
    assert_close(lse.cpu().numpy(), L, TOL_LSE["bf16"], "gqa_decode LSE")


def test_decode_equals_last_causal_row():
    """Decode of the last token equals the last row of a causal prefill."""
    B, Hq, Hkv, S, d = 1, 8, 2, 700, 128
    dev, _ = inputs(B, Hq, Hkv, S, S, d, "bf16", 55)
    of, lf = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    od, ld = aos.attn_decode(dev["q"][:, :, -1:].contiguous(), dev["k"], dev["v"], n_splits=16)
    torch.cuda.synchronize()
    assert_close(to_f64(od), to_f64(of[:, :, -1:]), 2e-2, "decode vs prefill last row")
    assert_close(ld.cpu().numpy(), lf[:, :, -1:].cpu().numpy(), 1e-3, "decode vs prefill LSE")


def test_decode_integrity():
    B, Hq, Hkv, Skv, d = 2, 8, 2, 999, 128
    dev, _ = inputs(B, Hq, Hkv, 1, Skv, d, "bf16", 66)
    keep = {k: v.clone() for k, v in dev.items()}
    o = torch.full_like(dev["q"], float("nan"))
    lse = torch.full((B, Hq, 1), float("nan"), device="cuda")
    ws = torch.full((aos.attn_decode_workspace_bytes(B, Hq, d, 16) // 4,), float("nan"),
                    device="cuda")
    note("decode integrity")
    aos.attn_decode(dev["q"], dev["k"], dev["v"], n_splits=16, o=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item()
    for k in dev:
        assert torch.equal(dev[k], keep[k]), f"input {k} mutated"
    o2, l2 = aos.attn_decode(dev["q"], dev["k"], dev["v"], n_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2)
    for name in ("q", "k", "v"):
        pert = {k: v.clone() for k, v in dev.items()}
        pert[name][1, 1, -1, 7] += 2.0
        o3, _ = aos.attn_decode(pert["q"], pert["k"], pert["v"], n_splits=16)
        torch.cuda.synchronize()
        assert not torch.equal(o3, o), f"output does not depend on {name}"
