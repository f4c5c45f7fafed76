"""Host-side parts of bench.py, on the CPU: the algorithmic work it divides
by the measured time (the roofline's `achieved`), the counter-summary gate
on `traffic`, and the one-GPU refusal.  The expected figures are the
configurations' own: allowed pairs counted by brute force over the mask
(small sizes) or by the closed form S(S+1)/2 for a causal square."""
import os
import shutil
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from attention_online_softmax_amd.inputs import WORKLOADS  # noqa: E402


def test_pairs_per_head_brute_force():
    """The allowed-pair count behind every FLOP figure, against the mask
    written out (bottom-right causal alignment, Sq <= Skv)."""
    from dataclasses import replace
    w0 = WORKLOADS["block_fwd"]
    for sq, skv, causal in ((7, 7, True), (5, 9, True), (33, 70, True), (6, 11, False)):
        w = replace(w0, Sq=sq, Skv=skv, causal=causal)
        i = np.arange(sq)[:, None]
        j = np.arange(skv)[None, :]
        allowed = (j <= i + (skv - sq)) if causal else np.ones((sq, skv), bool)
        assert w.pairs_per_head() == int(allowed.sum())


def test_training_step_work():
    """B4 H16 S2048 d128 causal: the forward 4 d FLOP per allowed pair
    (6.875e10), dK/dV 8 d (1.375e11), dQ 2 d; forward + backward 2.406e11."""
    w = WORKLOADS["train_fwd_bwd"]
    pairs = 2048 * 2049 // 2 * 4 * 16
    k = bench.per_kernel_algorithmic(w)
    assert k["fwd_bf16_kernel"] == ("mfma", 4.0 * 128 * pairs)
    assert k["bwd_dkdv_kernel"] == ("mfma", 8.0 * 128 * pairs)
    assert k["bwd_dq_kernel"] == ("mfma", 2.0 * 128 * pairs)
    total = sum(v[1] for v in k.values())
    assert abs(total - 2.406e11) / 2.406e11 < 1e-3
    assert abs(bench.flops_fwd(w) - 6.875e10) / 6.875e10 < 1e-3


def test_other_config_work():
    assert abs(bench.flops_fwd(WORKLOADS["block_fwd"]) - 2.152e9) / 2.152e9 < 1e-3
    assert abs(bench.flops_fwd(WORKLOADS["long_prefill"]) - 1.588e13) / 1.588e13 < 1e-3
    assert bench.flops_fwd(WORKLOADS["fp32_small"]) == 4.0 * 64 * 128 * 128


def test_decode_bytes():
    """The split kernel reads K and V once (2 x 8 x 8 x 4096 x 128 x 2 B =
    134.2 MB) and Q, and writes the 16 splits' states; the combine reads the
    states (and the query shape) and writes O and LSE."""
    w = WORKLOADS["gqa_decode"]
    k = bench.per_kernel_algorithmic(w)
    kv = 2 * 8 * 8 * 4096 * 128 * 2
    q = 8 * 32 * 128 * 2
    states = 16 * 8 * 32 * (128 + 2) * 4
    assert k["decode_split_kernel"] == ("hbm", float(kv + q + states))
    assert k["decode_combine_kernel"] == ("hbm", float(states + q + 8 * 32 * 4))
    assert abs(kv - 134.2e6) / 134.2e6 < 1e-3


def test_traffic_gate(tmp_path, monkeypatch):
    """A counter summary counts only while its source hash matches the
    kernel's current source: copy one, then change the copy's source."""
    src = os.path.join(ROOT, "profiles", "traffic_bwd_dkdv_kernel_train_fwd_bwd.txt")
    if not os.path.exists(src):
        pytest.skip("no committed counter summary for the dK/dV kernel")
    csrc = tmp_path / "attention_online_softmax_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in ("bwd_kernels.h", "common.h"):
        shutil.copy(os.path.join(ROOT, "attention_online_softmax_amd", "csrc", f), csrc / f)
    (tmp_path / "profiles").mkdir()
    text = open(src).read()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash("bwd_dkdv_kernel")
    lines = [("source_sha256_16: " + h) if l.startswith("source_sha256_16:") else l
             for l in text.splitlines()]
    dst = tmp_path / "profiles" / "traffic_bwd_dkdv_kernel_train_fwd_bwd.txt"
    dst.write_text("\n".join(lines) + "\n")
    v = bench.stored_traffic("bwd_dkdv_kernel", "train_fwd_bwd")
    assert v is not None and v > 0
    (csrc / "bwd_kernels.h").write_text((csrc / "bwd_kernels.h").read_text() + "\n// edited\n")
    assert bench.stored_traffic("bwd_dkdv_kernel", "train_fwd_bwd") is None
    assert bench.stored_traffic("bwd_dkdv_kernel", "no_such_workload") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="a GPU is present: bench.py would run")
def test_no_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr and r.stdout == ""
