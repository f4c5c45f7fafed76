"""Shared helpers for the GPU tests (parity against the oracle)."""
import sys

import numpy as np
import torch

from attention_online_softmax_amd.inputs import make_qkv, to_f64

# Tolerances: max-abs error against the float64 oracle.
TOL_O = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = {"f32": 1e-5, "bf16": 1e-3}
TOL_GRAD = 5e-2


def note(msg):
    """Print and flush what the next GPU step is, so a hang names its case."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(dt):
    return torch.float32 if dt == "f32" else torch.bfloat16


def inputs(B, Hq, Hkv, Sq, Skv, d, dt, seed, mult=1.0, with_do=False):
    cpu = make_qkv(B, Hq, Hkv, Sq, Skv, d, torch_dtype(dt), seed, mult, with_do)
    dev = {k: v.to("cuda") for k, v in cpu.items()}
    ref = {k: to_f64(v) for k, v in cpu.items()}
    return dev, ref


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite values in GPU output"
    return float(np.max(np.abs(a - b)))


def assert_close(gpu, ref, tol, what):
    err = max_abs(gpu, ref)
    note(f"{what}: max abs err {err:.3e} (tol {tol:.1e})")
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
