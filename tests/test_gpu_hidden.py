"""Hidden-semantics inputs through the C ABI against the float64 oracle.

"Compilers and Kernels", section "Generated kernels need a hostile
evaluator", item 2: the inputs a kernel author is least likely to have tried
-- large-magnitude scores, zero and negative-zero inputs, ties, a dominant key
that arrives late in a row's key loop, negative, zero and negative-zero
scales -- on every entry point and every kernel family (fp32 and bf16
forward at d = 64, 128, 256, causal and not; the matrix-core, vector-unit and
paged decodes; the two-kernel and fused backwards).

Tolerances.  The parity tolerances (fp32 O 1e-5, bf16 O 2e-2, gradients
5e-2; LSE 1e-5 / 1e-3 by our reading) are absolute and hold for values of
unit size.  These inputs make scores, LSE and gradients far larger, so the
tolerances add what the dtypes themselves force:
* scores: the kernels form every score in fp32, so an exponent argument of
  size |s| carries a rounding error of up to about
  delta = (4 + sqrt(d)) * 2 * 2^-24 * max|s| (the dot product's
  accumulation, the scale, the log2(e) factor, the subtraction of the row
  reference).  LSE is of the size of the scores and moves by up to delta:
  its tolerance is the base plus delta for every kind.  A perturbation of
  at most delta in every score moves each softmax weight by a factor within
  exp(+-2 delta), so O moves by at most 2 delta max|V|; that worst case is
  added for the large-magnitude kind (for unit-size inputs it stays below
  the base tolerance in practice and is left out).
* gradients: they are stored in bf16, whose rounding alone is up to 2^-8 of
  the value, and P and dS are rounded to bf16 before their products (another
  2^-8 relative); the tolerance adds (2^-7 + 2 delta) max|reference
  gradient| (a gradient of 58 has a half ulp of 0.125 > 5e-2).
"""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import make_paged, randn, to_f64
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, max_abs, note, torch_dtype

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24

KINDS = ["x30", "zero_q", "negzero_q", "tied_keys", "late_dominant", "neg_scale", "zero_scale",
         "negzero_scale"]


def hostile(kind, B, Hq, Hkv, Sq, Skv, d, dt, seed, with_do=False):
    """Seeded CPU inputs of one hidden-semantics kind and the scale to use.

    x30: Q, K, V (not dO) N(0,1) * 30, scores about 900 times their usual
      size;
    zero_q / negzero_q: Q all +0 / all -0 (uniform weights: the mean of the
      allowed values);
    tied_keys: every key row of a head equal (uniform weights again);
    late_dominant: Q column 0 = 4, K column 0 = 0 except three planted keys
      at Skv/3, 2 Skv/3 and Skv - 5 (the last 32-key tile) whose scores rise
      by about 15, 30 and 45: each one passes the running maximum by more
      than the lazy-rescale threshold, late in the rows that see it;
    neg_scale / zero_scale / negzero_scale: N(0,1) inputs with scale
      -1/sqrt(d), 0 and -0.0.
    """
    tdt = torch_dtype(dt)
    mult = 30.0 if kind == "x30" else 1.0
    q = randn((B, Hq, Sq, d), seed, mult, torch.float32)
    k = randn((B, Hkv, Skv, d), seed + 1, mult, torch.float32)
    v = randn((B, Hkv, Skv, d), seed + 2, mult, torch.float32)
    scale = 1.0 / math.sqrt(d)
    if kind == "zero_q":
        q.zero_()
    elif kind == "negzero_q":
        q.fill_(-0.0)
    elif kind == "tied_keys":
        k[:] = k[:, :, :1, :]
    elif kind == "late_dominant":
        q.mul_(0.5)
        k.mul_(0.5)
        q[..., 0] = 4.0
        k[..., 0] = 0.0
        for pos, boost in ((Skv // 3, 15.0), (2 * Skv // 3, 30.0), (Skv - 5, 45.0)):
            if 0 <= pos < Skv:
                k[:, :, pos, 0] = boost * math.sqrt(d) / 4.0
    elif kind == "neg_scale":
        scale = -scale
    elif kind == "zero_scale":
        scale = 0.0
    elif kind == "negzero_scale":
        scale = -0.0
    out = {"q": q.to(tdt), "k": k.to(tdt), "v": v.to(tdt)}
    if with_do:
        out["do"] = randn((B, Hq, Sq, d), seed + 3, 1.0, tdt)
    return out, scale


def score_delta(ref, scale, d):
    """Bound on the fp32 rounding of an exponent argument (natural-log
    units): (4 + sqrt(d)) * 2 * 2^-24 * max |scale q_i . k_j| over all pairs."""
    q, k = ref["q"], ref["k"]
    B, Hq, Sq, _ = q.shape
    G = Hq // k.shape[1]
    smax = 0.0
    for b in range(B):
        for h in range(Hq):
            s = np.abs(q[b, h] @ k[b, h // G].T) * abs(scale)
            smax = max(smax, float(s.max()) if s.size else 0.0)
    return (4.0 + math.sqrt(d)) * 2.0 * U32 * smax


def tols(kind, dt, ref, scale, d):
    """(O, LSE) tolerances and delta, as derived in the module docstring."""
    delta = score_delta(ref, scale, d)
    tol_o = TOL_O[dt]
    if kind == "x30":
        tol_o += 2 * delta * float(np.abs(ref["v"]).max())
    return tol_o, TOL_LSE[dt] + delta, delta


def check(got_o, got_l, O, L, tol_o, tol_l, what):
    """O and LSE against the oracle; rows with no allowed key (oracle LSE
    -inf, possible with a bias) must have O = 0 and LSE = -inf."""
    got_o = np.asarray(got_o, dtype=np.float64)
    got_l = np.asarray(got_l, dtype=np.float64).reshape(L.shape)
    dead = np.isinf(L)
    assert np.array_equal(np.isneginf(got_l), dead), f"{what}: rows without keys differ"
    assert np.all(got_o[dead] == 0), f"{what}: O of a row without keys"
    assert np.all(np.isfinite(got_o)), f"{what}: non-finite O"
    eo = max_abs(got_o, O)
    el = max_abs(np.where(dead, 0.0, got_l), np.where(dead, 0.0, L))
    note(f"{what}: O err {eo:.3e} (tol {tol_o:.2e}), LSE err {el:.3e} (tol {tol_l:.2e})")
    assert eo <= tol_o, f"{what}: O max abs err {eo:.3e} > {tol_o:.2e}"
    assert el <= tol_l, f"{what}: LSE max abs err {el:.3e} > {tol_l:.2e}"


def ids(c):
    return "_".join(str(x) for x in c)


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------
FWD = [(dt, d, causal, kind) for dt in ("f32", "bf16") for d in (64, 128, 256)
       for causal in (True, False) for kind in KINDS]


@pytest.mark.parametrize("case", FWD, ids=ids)
def test_fwd_hidden(case):
    dt, d, causal, kind = case
    B, Hq, Hkv, S = 1, 2, 1, 300
    cpu, scale = hostile(kind, B, Hq, Hkv, S, S, d, dt, 7000 + d + 2 * causal)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"fwd hidden {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    tol_o, tol_l, _ = tols(kind, dt, ref, scale, d)
    check(to_f64(o), lse.cpu().numpy(), O, L, tol_o, tol_l, f"fwd {case}")


# The bf16 forward's tiles forced one by one on every kind: the key-split
# kernel (every wave of a workgroup on one 32-row block, each with its own
# keys), two key groups sharing their query blocks, and a plain tile; the
# groups' states are merged at the end.  The estimate picks among them by
# grid size, so no family's hidden-semantics coverage is left to it.
FWD_TILES = [(d, causal, kind, nw, bc, sp) for d in (64, 128) for causal in (True, False)
             for kind in KINDS
             for nw, bc, sp in ((4, 32, 4), (2, 32, 2), (4, 32, 1), (4, 64 if d == 64 else 32, 2))]


@pytest.mark.parametrize("case", FWD_TILES, ids=ids)
def test_fwd_hidden_forced_tile(case):
    d, causal, kind, nw, bc, sp = case
    B, Hq, Hkv, Sq, Skv = 1, 2, 1, 300, 333
    cpu, scale = hostile(kind, B, Hq, Hkv, Sq, Skv, d, "bf16", 7300 + d + 2 * causal)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"fwd hidden forced tile {case}")
    aos.attn_fwd_tile_override(nw, bc, sp)
    try:
        o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
        torch.cuda.synchronize()
    finally:
        aos.attn_fwd_tile_override(0, 0)
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    tol_o, tol_l, _ = tols(kind, "bf16", ref, scale, d)
    check(to_f64(o), lse.cpu().numpy(), O, L, tol_o, tol_l, f"fwd forced {case}")


# A 256-thread-workgroup fp32 grid (32 columns per lane) and bf16 grids with
# several workgroups per head, for the kinds that stress the softmax.
FWD_LARGE = [(dt, d, kind) for dt, d in (("f32", 64), ("bf16", 128), ("bf16", 64))
             for kind in ("x30", "late_dominant", "zero_scale", "neg_scale")]


@pytest.mark.parametrize("case", FWD_LARGE, ids=ids)
def test_fwd_hidden_large_grid(case):
    dt, d, kind = case
    B, Hq, Hkv, S = 2, 64, 16, 200
    cpu, scale = hostile(kind, B, Hq, Hkv, S, S, d, dt, 7100 + d)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"fwd hidden large grid {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale)
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, scale)
    tol_o, tol_l, _ = tols(kind, dt, ref, scale, d)
    check(to_f64(o), lse.cpu().numpy(), O, L, tol_o, tol_l, f"fwd large {case}")


# Additive bias and sliding window with zero and negative scales: the bias
# alone then decides the weights (zero scale), or the scores change sign.
BIAS_CASES = [(dt, d, kind, window) for dt, d in (("f32", 64), ("bf16", 64), ("bf16", 128),
                                                  ("bf16", 256))
              for kind in ("zero_scale", "neg_scale", "negzero_scale") for window in (0, 50)]


@pytest.mark.parametrize("case", BIAS_CASES, ids=ids)
def test_fwd_hidden_bias_window(case):
    from tests.test_gpu_bias import make_bias
    dt, d, kind, window = case
    B, Hq, Hkv, S = 2, 2, 1, 150
    cpu, scale = hostile(kind, B, Hq, Hkv, S, S + 2, d, dt, 7200 + d)
    bias = make_bias("full", B, Hq, S, S + 2, 7250 + d)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"fwd hidden bias/window {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True, scale=scale, window=window,
                          bias=bias.cuda())
    torch.cuda.synchronize()
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], True, scale, window=window,
                                bias=bias.numpy().astype(np.float64))
    check(to_f64(o), lse.cpu().numpy(), O, L, TOL_O[dt], TOL_LSE[dt], f"fwd bias {case}")


# ---------------------------------------------------------------------------
# Decode: matrix-core kernel (bf16 d64, d128), vector-unit kernel (fp32, bf16
# d256), 1000 keys (a ragged last 32-key tile), 16 and 5 splits.
# ---------------------------------------------------------------------------
DEC = [(dt, d, n, kind) for dt, d in (("bf16", 64), ("bf16", 128), ("bf16", 256), ("f32", 64),
                                      ("f32", 128))
       for n in (16, 5) for kind in KINDS]


@pytest.mark.parametrize("case", DEC, ids=ids)
def test_decode_hidden(case):
    dt, d, n, kind = case
    B, Hq, Hkv, Skv = 2, 8, 2, 1000
    cpu, scale = hostile(kind, B, Hq, Hkv, 1, Skv, d, dt, 7300 + d + n)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"decode hidden {case}")
    o, lse = aos.attn_decode(dev["q"], dev["k"], dev["v"], scale=scale, n_splits=n)
    torch.cuda.synchronize()
    O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], scale, n)
    tol_o, tol_l, _ = tols(kind, dt, ref, scale, d)
    check(to_f64(o), lse.cpu().numpy(), O, L, tol_o, tol_l, f"decode {case}")


PAGED = [(d, kind) for d in (64, 128) for kind in KINDS]


@pytest.mark.parametrize("case", PAGED, ids=ids)
def test_decode_paged_hidden(case):
    """Paged decode: the kind's query and keys poured into shuffled 64-key
    pages, ragged stream lengths."""
    d, kind = case
    B, Hq, Hkv, ps, mp = 3, 8, 2, 64, 16
    lens = [1000, 777, 64]
    cpu, scale = hostile(kind, B, Hq, Hkv, 1, mp * ps, d, "bf16", 7400 + d)
    pg = make_paged(B, Hq, Hkv, d, ps, mp, lens, seed=7450 + d)
    # Stream b's key t is row t % ps of page table[b][t // ps].
    kp, vp = pg["k_pages"].clone(), pg["v_pages"].clone()
    table = pg["block_table"]
    for b in range(B):
        for p in range(mp):
            kp[table[b, p]] = cpu["k"][b, :, p * ps:(p + 1) * ps]
            vp[table[b, p]] = cpu["v"][b, :, p * ps:(p + 1) * ps]
    pg.update(q=cpu["q"], k_pages=kp, v_pages=vp)
    dev = {k: v.cuda() for k, v in pg.items()}
    note(f"decode paged hidden {case}")
    o, lse = aos.attn_decode_paged(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                                   dev["seq_lens"], scale=scale, n_splits=16)
    torch.cuda.synchronize()
    ref = {k: (to_f64(v) if v.is_floating_point() else v.numpy()) for k, v in pg.items()}
    O, L = oracle.decode_paged_ref(ref["q"], ref["k_pages"], ref["v_pages"], ref["block_table"],
                                   ref["seq_lens"], scale)
    qkv = {"q": ref["q"], "k": to_f64(cpu["k"]), "v": to_f64(cpu["v"])}
    tol_o, tol_l, _ = tols(kind, "bf16", qkv, scale, d)
    check(to_f64(o), lse.cpu().numpy(), O, L, tol_o, tol_l, f"paged {case}")


# ---------------------------------------------------------------------------
# Backward (two-kernel and fused), bf16 d64 and d128; the two-kernel one
# also at d256.  The shape is small enough that the library takes the
# grouped launch shapes of both backward kernels; "plain" holds them to the
# plain (4, 1) shapes instead.
# ---------------------------------------------------------------------------
BWD = ([(mode, d, causal, kind) for mode in ("picked", "fused") for d in (64, 128, 256)
        for causal in (True, False) for kind in KINDS if not (mode == "fused" and d == 256)] +
       [("plain", d, causal, kind) for d in (64, 128) for causal in (True, False)
        for kind in KINDS])


@pytest.mark.parametrize("case", BWD, ids=lambda c: ("" if c[0] == "picked" else c[0] + "_") +
                         ids(c[1:]))
def test_bwd_hidden(case):
    mode, d, causal, kind = case
    B, Hq, Hkv, Sq, Skv = 1, 2, 1, 200, 230
    cpu, scale = hostile(kind, B, Hq, Hkv, Sq, Skv, d, "bf16", 7500 + d + causal, with_do=True)
    ref = {k: to_f64(v) for k, v in cpu.items()}
    dev = {k: v.cuda() for k, v in cpu.items()}
    note(f"bwd hidden {case}")
    o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
    bwd = aos.attn_bwd_fused if mode == "fused" else aos.attn_bwd
    if mode == "plain":
        aos.attn_bwd_tile_override(4, 1, 4, 1, 1)
    try:
        dq, dk, dv = bwd(dev["q"], dev["k"], dev["v"], o, dev["do"], lse, causal=causal,
                         scale=scale)
        torch.cuda.synchronize()
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0)
    rq, rk, rv, _ = oracle.attention_bwd_ref(ref["q"], ref["k"], ref["v"], ref["do"], causal,
                                             scale)
    _, _, delta = tols(kind, "bf16", ref, scale, d)
    for name, got, want in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
        g = to_f64(got)
        assert np.all(np.isfinite(g)), f"{name}: non-finite"
        tol = TOL_GRAD + (2.0 ** -7 + 2 * delta) * float(np.abs(want).max())
        err = max_abs(g, want)
        note(f"bwd {case} {name}: err {err:.3e} (tol {tol:.2e}, max |ref| "
             f"{float(np.abs(want).max()):.3g})")
        assert err <= tol, f"{name}: max abs err {err:.3e} > {tol:.2e}"
