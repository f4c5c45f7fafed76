"""Out-of-bounds detection with guard regions ("Compilers and Kernels",
section "Generated kernels need a hostile evaluator", item 3: detect
out-of-bounds access).

Every output and every workspace is carved out of the middle of a larger
device buffer whose guard bytes before and after it hold a known pattern;
after the call the guards must be unchanged, byte for byte, so a write past
either end of an output (a ragged tail, a padded row, a split state) is
caught.  Every input sits between guards of NaN: a read past an input that
reaches the result turns it NaN, and the outputs must be finite and match the
oracle.  Shapes are ragged (rows and keys not multiples of the tiles) so the
last tiles of every kernel are partial.
"""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import make_paged, make_qkv, randn, to_f64
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, assert_close, note, torch_dtype

pytestmark = pytest.mark.gpu

GUARD = 4096   # bytes of guard before and after each buffer (a multiple of 16)
PATTERN = 0xA5


class Guarded:
    """A contiguous tensor of `shape` placed GUARD bytes into a device byte
    buffer; the guard bytes hold PATTERN (outputs, workspaces) or NaN
    (inputs)."""

    def __init__(self, shape, dtype, fill_nan=False, init=None):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) if len(shape) else 1
        self.nbytes = n * esz
        self.buf = torch.full((GUARD + self.nbytes + GUARD,), PATTERN, dtype=torch.uint8,
                              device="cuda")
        if fill_nan:
            assert dtype in (torch.float32, torch.bfloat16)
            nan = torch.full((self.buf.numel() // esz,), float("nan"), dtype=dtype, device="cuda")
            self.buf.copy_(nan.view(torch.uint8))
        self.t = self.buf[GUARD:GUARD + self.nbytes].view(dtype).view(*shape)
        if init is not None:
            self.t.copy_(init)
        self.before = self.buf[:GUARD].clone()
        self.after = self.buf[GUARD + self.nbytes:].clone()

    def check(self, what):
        assert torch.equal(self.buf[:GUARD], self.before), f"{what}: write before the buffer"
        assert torch.equal(self.buf[GUARD + self.nbytes:], self.after), \
            f"{what}: write past the end of the buffer"


def guarded_inputs(cpu):
    return {k: Guarded(tuple(v.shape), v.dtype, fill_nan=v.is_floating_point(), init=v.cuda())
            for k, v in cpu.items()}


def workspace(nbytes):
    return Guarded((nbytes,), torch.uint8)


FWD = [("f32", 64, 200, 200, True), ("f32", 128, 77, 301, False), ("f32", 256, 65, 65, True),
       ("bf16", 64, 200, 200, True), ("bf16", 128, 300, 333, True), ("bf16", 128, 97, 161, False),
       ("bf16", 256, 130, 130, True), ("bf16", 256, 1, 777, False)]


@pytest.mark.parametrize("case", FWD, ids=lambda c: "_".join(map(str, c)))
def test_fwd_guards(case):
    dt, d, Sq, Skv, causal = case
    B, Hq, Hkv = 2, 4, 2
    cpu = make_qkv(B, Hq, Hkv, Sq, Skv, d, torch_dtype(dt), seed=8000 + d + Sq)
    gin = guarded_inputs(cpu)
    go = Guarded((B, Hq, Sq, d), torch_dtype(dt))
    gl = Guarded((B, Hq, Sq), torch.float32)
    scale = 1 / math.sqrt(d)
    note(f"fwd guards {case}")
    aos.attn_fwd(gin["q"].t, gin["k"].t, gin["v"].t, causal=causal, scale=scale, o=go.t, lse=gl.t)
    torch.cuda.synchronize()
    go.check("O")
    gl.check("LSE")
    for k, g in gin.items():
        g.check(f"input {k}")
    ref = {k: to_f64(v) for k, v in cpu.items()}
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    assert_close(to_f64(go.t), O, TOL_O[dt], "O")
    assert_close(gl.t.cpu().numpy(), L, TOL_LSE[dt], "LSE")


def test_fwd_bias_window_guards():
    """bf16 and f32 forward with a sliding window and a guarded bias whose
    rows are not a multiple of the key tile."""
    from tests.test_gpu_bias import make_bias
    for dt in ("bf16", "f32"):
        B, Hq, Hkv, Sq, Skv, d, W = 2, 2, 1, 150, 164, 64, 40
        cpu = make_qkv(B, Hq, Hkv, Sq, Skv, d, torch_dtype(dt), seed=8100)
        bias = make_bias("full", B, Hq, Sq, Skv, 8101)
        gin = guarded_inputs(cpu)
        gb = Guarded(tuple(bias.shape), torch.float32, fill_nan=True, init=bias.cuda())
        go = Guarded((B, Hq, Sq, d), torch_dtype(dt))
        gl = Guarded((B, Hq, Sq), torch.float32)
        note(f"fwd bias/window guards {dt}")
        aos.attn_fwd(gin["q"].t, gin["k"].t, gin["v"].t, causal=True, scale=0.125, o=go.t,
                     lse=gl.t, window=W, bias=gb.t)
        torch.cuda.synchronize()
        go.check("O")
        gl.check("LSE")
        gb.check("bias")
        ref = {k: to_f64(v) for k, v in cpu.items()}
        O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, 0.125, window=W,
                                    bias=bias.numpy().astype(np.float64))
        dead = np.isinf(L)
        got_l = gl.t.cpu().numpy()
        assert np.array_equal(np.isneginf(got_l), dead)
        assert_close(to_f64(go.t), O, TOL_O[dt], f"{dt} O")
        assert_close(np.where(dead, 0, got_l), np.where(dead, 0, L), TOL_LSE[dt], f"{dt} LSE")


DEC = [("bf16", 128, 1000, 16), ("bf16", 64, 513, 7), ("bf16", 256, 300, 5), ("f32", 64, 999, 16),
       ("f32", 128, 37, 16)]


@pytest.mark.parametrize("case", DEC, ids=lambda c: "_".join(map(str, c)))
def test_decode_guards(case):
    dt, d, Skv, n = case
    B, Hq, Hkv = 2, 8, 2
    cpu = make_qkv(B, Hq, Hkv, 1, Skv, d, torch_dtype(dt), seed=8200 + d + n)
    gin = guarded_inputs(cpu)
    go = Guarded((B, Hq, 1, d), torch_dtype(dt))
    gl = Guarded((B, Hq, 1), torch.float32)
    gw = workspace(aos.attn_decode_workspace_bytes(B, Hq, d, n))
    scale = 1 / math.sqrt(d)
    note(f"decode guards {case}")
    aos.attn_decode(gin["q"].t, gin["k"].t, gin["v"].t, scale=scale, n_splits=n, o=go.t, lse=gl.t,
                    workspace=gw.t)
    torch.cuda.synchronize()
    go.check("O")
    gl.check("LSE")
    gw.check("workspace")
    ref = {k: to_f64(v) for k, v in cpu.items()}
    O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], scale, n)
    assert_close(to_f64(go.t), O, TOL_O[dt], "decode O")
    assert_close(gl.t.cpu().numpy(), L, TOL_LSE[dt], "decode LSE")


@pytest.mark.parametrize("d", [64, 128])
def test_decode_paged_guards(d):
    """Guarded pools, table and lengths; one table entry points past the pool
    (read as zeros, never outside the pools)."""
    B, Hq, Hkv, ps, mp = 3, 8, 2, 64, 6
    cpu = make_paged(B, Hq, Hkv, d, ps, mp, [300, 65, 0], seed=8300 + d)
    cpu["block_table"][0, 2] = cpu["k_pages"].shape[0] + 5
    gin = {k: Guarded(tuple(v.shape), v.dtype, fill_nan=v.is_floating_point(), init=v.cuda())
           for k, v in cpu.items()}
    go = Guarded((B, Hq, 1, d), torch.bfloat16)
    gl = Guarded((B, Hq, 1), torch.float32)
    gw = workspace(aos.attn_decode_workspace_bytes(B, Hq, d, 16))
    scale = 1 / math.sqrt(d)
    note(f"decode paged guards d{d}")
    aos.attn_decode_paged(gin["q"].t, gin["k_pages"].t, gin["v_pages"].t, gin["block_table"].t,
                          gin["seq_lens"].t, scale=scale, n_splits=16, o=go.t, lse=gl.t,
                          workspace=gw.t)
    torch.cuda.synchronize()
    for name, g in [("O", go), ("LSE", gl), ("workspace", gw)] + list(gin.items()):
        g.check(name)
    ref = {k: (to_f64(v) if v.is_floating_point() else v.numpy()) for k, v in cpu.items()}
    O, L = oracle.decode_paged_ref(ref["q"], ref["k_pages"], ref["v_pages"], ref["block_table"],
                                   ref["seq_lens"], scale)
    got_l = gl.t.cpu().numpy()
    empty = np.isinf(L)
    assert np.array_equal(np.isneginf(got_l), empty)
    assert_close(to_f64(go.t), O, TOL_O["bf16"], "paged O")
    assert_close(np.where(empty, 0, got_l), np.where(empty, 0, L), TOL_LSE["bf16"], "paged LSE")


BWD = [(False, 64, 130, 300, True), (False, 128, 200, 200, True), (False, 128, 97, 161, False),
       (True, 64, 130, 300, True), (True, 128, 97, 161, False)]


@pytest.mark.parametrize("case", BWD, ids=lambda c: ("fused_" if c[0] else "") +
                         "_".join(map(str, c[1:])))
def test_bwd_guards(case):
    fused, d, Sq, Skv, causal = case
    B, Hq, Hkv = 2, 4, 2
    cpu = make_qkv(B, Hq, Hkv, Sq, Skv, d, torch.bfloat16, seed=8400 + d + Sq, with_do=True)
    scale = 1 / math.sqrt(d)
    dev = {k: v.cuda() for k, v in cpu.items()}
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    cpu2 = dict(cpu, o=o.cpu(), lse=lse.cpu())
    gin = guarded_inputs(cpu2)
    gq = Guarded((B, Hq, Sq, d), torch.bfloat16)
    gk = Guarded((B, Hkv, Skv, d), torch.bfloat16)
    gv = Guarded((B, Hkv, Skv, d), torch.bfloat16)
    wsb = (aos.attn_bwd_fused_workspace_bytes if fused else aos.attn_bwd_workspace_bytes)(
        B, Hq, Sq, d)
    gw = workspace(wsb)
    bwd = aos.attn_bwd_fused if fused else aos.attn_bwd
    note(f"bwd guards {case}")
    bwd(gin["q"].t, gin["k"].t, gin["v"].t, gin["o"].t, gin["do"].t, gin["lse"].t, causal=causal,
        scale=scale, dq=gq.t, dk=gk.t, dv=gv.t, workspace=gw.t)
    torch.cuda.synchronize()
    for name, g in [("dQ", gq), ("dK", gk), ("dV", gv), ("workspace", gw)] + list(gin.items()):
        g.check(name)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal, scale)
    assert_close(to_f64(gq.t), rq, TOL_GRAD, "dQ")
    assert_close(to_f64(gk.t), rk, TOL_GRAD, "dK")
    assert_close(to_f64(gv.t), rv, TOL_GRAD, "dV")
