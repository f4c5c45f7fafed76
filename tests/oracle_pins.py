"""Pins for the float64 oracle: checks against things other than the oracle.

Each `pin_*` function takes the oracle module `A` (so the mutation tests can
hand it a copy with a planted mistake) and raises AssertionError on mismatch.
The sources of truth are: mpmath brute force with 50 digits and no max shift,
the hand-worked rational example under tests/golden/, closed forms (uniform
scores, one-hot scores, a single key), library routines (scipy logsumexp and
softmax, torch float64 scaled_dot_product_attention and autograd), exact
invariants (key shift, key permutation, grouped heads as repeated heads,
decode as the last causal row) and central finite differences.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import mpmath
import numpy as np
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(seed, *shape, mult=1.0):
    return _rng(seed).standard_normal(shape) * mult


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _allowed(i, Sq, Skv, causal):
    return Skv if not causal else min(i + Skv - Sq + 1, Skv)


# ---------------------------------------------------------------- forward

def _mp_attention(q, k, v, causal, scale):
    """50-digit softmax attention written without the max shift: O_i =
    sum_j e^{S_ij} v_j / sum_j e^{S_ij}, LSE_i = ln sum_j e^{S_ij}."""
    mpmath.mp.dps = 50
    B, Hq, Sq, d = q.shape
    Hkv, Skv, dv = k.shape[1], k.shape[2], v.shape[3]
    g = Hq // Hkv
    O = np.zeros((B, Hq, Sq, dv))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for i in range(Sq):
                n = _allowed(i, Sq, Skv, causal)
                num = [mpmath.mpf(0)] * dv
                den = mpmath.mpf(0)
                for j in range(n):
                    s = mpmath.mpf(0)
                    for c in range(d):
                        s += mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, kh, j, c])
                    e = mpmath.exp(s * mpmath.mpf(scale))
                    den += e
                    for c in range(dv):
                        num[c] += e * mpmath.mpf(v[b, kh, j, c])
                for c in range(dv):
                    O[b, h, i, c] = float(num[c] / den)
                L[b, h, i] = float(mpmath.log(den))
    return O, L


def pin_fwd_mpmath(A):
    """Brute force at 50 digits on tiny shapes, causal and not, with GQA and
    Sq < Skv (bottom-right causal alignment)."""
    for seed, (B, Hq, Hkv, Sq, Skv, d), causal in [
        (1, (1, 2, 1, 3, 5, 3), True),
        (2, (2, 2, 2, 4, 4, 2), False),
        (3, (1, 4, 2, 2, 6, 4), True),
        (4, (1, 1, 1, 5, 5, 3), True),
    ]:
        q = _rand(seed, B, Hq, Sq, d)
        k = _rand(seed + 10, B, Hkv, Skv, d)
        v = _rand(seed + 20, B, Hkv, Skv, d)
        scale = 0.7
        O, L = A.attention_ref(q, k, v, causal, scale)
        Om, Lm = _mp_attention(q, k, v, causal, scale)
        _close(O, Om, 1e-13, "mpmath O")
        _close(L, Lm, 1e-13, "mpmath LSE")


def _golden():
    with open(os.path.join(GOLDEN, "rational_softmax.json")) as f:
        return json.load(f)


def _frac(x):
    return float(Fraction(x))


def _golden_qkv(w, V):
    n = len(w)
    q = np.zeros((1, 1, n, 2))
    q[..., 0] = 2.0
    k = np.zeros((1, 1, n, 2))
    k[0, 0, :, 0] = np.log(np.asarray(w, dtype=np.float64))
    v = np.asarray(V, dtype=np.float64)[None, None]
    return q, k, v


def pin_fwd_golden(A):
    """Hand-worked rational example (tests/golden/rational_softmax.json)."""
    gd = _golden()
    q, k, v = _golden_qkv(gd["w"], gd["V"])
    scale = _frac(gd["scale"])
    fw = gd["forward"]
    O, L = A.attention_ref(q, k, v, True, scale)
    _close(O[0, 0], [[_frac(x) for x in r] for r in fw["causal_O"]], 1e-14, "golden causal O")
    _close(L[0, 0], [math.log(_frac(x)) for x in fw["causal_LSE_exp"]], 1e-14, "golden causal LSE")
    O, L = A.attention_ref(q, k, v, False, scale)
    _close(O[0, 0], [[_frac(x) for x in fw["full_O_row"]]] * 4, 1e-14, "golden full O")
    _close(L[0, 0], [math.log(_frac(fw["full_LSE_exp"]))] * 4, 1e-14, "golden full LSE")


def pin_fwd_uniform(A):
    """Q = 0 makes every allowed score 0: O_i is the mean of the allowed V
    rows and LSE_i = ln(number of allowed keys)."""
    for causal, Sq, Skv in [(True, 7, 7), (True, 5, 9), (False, 4, 6)]:
        B, Hq, Hkv, d = 2, 4, 2, 3
        q = np.zeros((B, Hq, Sq, d))
        k = _rand(5, B, Hkv, Skv, d)
        v = _rand(6, B, Hkv, Skv, d)
        O, L = A.attention_ref(q, k, v, causal, 0.3)
        for b in range(B):
            for h in range(Hq):
                for i in range(Sq):
                    n = _allowed(i, Sq, Skv, causal)
                    _close(O[b, h, i], v[b, h // 2, :n].mean(axis=0), 1e-14, "uniform O")
                    _close(L[b, h, i], math.log(n), 1e-14, "uniform LSE")


def pin_fwd_onehot(A):
    """Scores set to chosen values: K_j = c_j e_0, Q_i = e_0 / scale gives
    S_ij = c_j. One score 40 above the rest selects its V row."""
    Skv, d = 9, 4
    scale = 0.25
    c = np.zeros(Skv)
    t = 6
    c[t] = 40.0
    k = np.zeros((1, 1, Skv, d))
    k[0, 0, :, 0] = c
    q = np.zeros((1, 1, 1, d))
    q[0, 0, 0, 0] = 1.0 / scale
    v = _rand(7, 1, 1, Skv, d)
    O, L = A.attention_ref(q, k, v, False, scale)
    _close(O[0, 0, 0], v[0, 0, t], 1e-14, "one-hot O")
    _close(L[0, 0, 0], 40.0 + math.log1p((Skv - 1) * math.exp(-40.0)), 1e-13, "one-hot LSE")


def pin_fwd_single_key(A):
    """A single key: O = V_0, LSE = scale q . k_0."""
    q = _rand(8, 1, 3, 1, 5)
    k = _rand(9, 1, 3, 1, 5)
    v = _rand(10, 1, 3, 1, 5)
    O, L = A.attention_ref(q, k, v, False, 0.9)
    _close(O, v, 1e-15, "single-key O")
    _close(L[..., 0], 0.9 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), 1e-14, "single-key LSE")


def pin_fwd_scipy(A):
    """Row by row with scipy.special.softmax / logsumexp on the masked scores."""
    B, Hq, Hkv, Sq, Skv, d = 1, 4, 2, 6, 11, 8
    q = _rand(11, B, Hq, Sq, d)
    k = _rand(12, B, Hkv, Skv, d)
    v = _rand(13, B, Hkv, Skv, d)
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        O, L = A.attention_ref(q, k, v, causal, scale)
        for h in range(Hq):
            kh = h // (Hq // Hkv)
            for i in range(Sq):
                n = _allowed(i, Sq, Skv, causal)
                s = np.array([scale * float(np.dot(q[0, h, i], k[0, kh, j])) for j in range(n)])
                p = scipy.special.softmax(s)
                _close(O[0, h, i], p @ v[0, kh, :n], 1e-14, "scipy O")
                _close(L[0, h, i], scipy.special.logsumexp(s), 1e-14, "scipy LSE")


def pin_fwd_torch_sdpa(A):
    """torch's float64 CPU scaled_dot_product_attention with an explicit
    bottom-right boolean mask and key/value heads repeated per group."""
    B, Hq, Hkv, Sq, Skv, d = 2, 6, 3, 13, 21, 16
    q = _rand(14, B, Hq, Sq, d)
    k = _rand(15, B, Hkv, Skv, d)
    v = _rand(16, B, Hkv, Skv, d)
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        O, _ = A.attention_ref(q, k, v, causal, scale)
        kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
        vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
        mask = None
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Skv)[None, :]
            mask = j <= i + (Skv - Sq)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), kt, vt, attn_mask=mask, scale=scale)
        _close(O, ref.numpy(), 1e-13, "torch sdpa O")


def pin_fwd_window(A):
    """Sliding windows of W keys ending at the diagonal: 50-digit brute force
    over exactly the keys j with i + off - W < j <= i + off; torch float64
    sdpa with that boolean mask; W = 1 selects the diagonal key (O = V,
    LSE = scale q . k); W at least Skv is the plain causal mask."""
    for seed, (B, Hq, Hkv, Sq, Skv, d), W in [(50, (1, 2, 1, 6, 6, 3), 3),
                                              (51, (1, 2, 2, 4, 9, 2), 4)]:
        q = _rand(seed, B, Hq, Sq, d)
        k = _rand(seed + 10, B, Hkv, Skv, d)
        v = _rand(seed + 20, B, Hkv, Skv, d)
        O, L = A.attention_ref(q, k, v, True, 0.6, window=W)
        mpmath.mp.dps = 50
        g = Hq // Hkv
        for b in range(B):
            for h in range(Hq):
                for i in range(Sq):
                    hi = i + Skv - Sq
                    js = range(max(0, hi - W + 1), hi + 1)
                    es = [mpmath.exp(mpmath.mpf(0.6) * mpmath.fsum(
                        mpmath.mpf(q[b, h, i, c]) * mpmath.mpf(k[b, h // g, j, c])
                        for c in range(d))) for j in js]
                    den = mpmath.fsum(es)
                    for c in range(d):
                        num = mpmath.fsum(e * mpmath.mpf(v[b, h // g, j, c]) for e, j in zip(es, js))
                        _close(O[b, h, i, c], float(num / den), 1e-13, "window mpmath O")
                    _close(L[b, h, i], float(mpmath.log(den)), 1e-13, "window mpmath LSE")
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 11, 17, 8
    q = _rand(52, B, Hq, Sq, d)
    k = _rand(53, B, Hkv, Skv, d)
    v = _rand(54, B, Hkv, Skv, d)
    scale = 1 / math.sqrt(d)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Skv)[None, :]
    for W in (1, 2, 5, Skv - 1):
        O, L = A.attention_ref(q, k, v, True, scale, window=W)
        mask = (j <= i + (Skv - Sq)) & (j > i + (Skv - Sq) - W)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), kt, vt, attn_mask=mask, scale=scale)
        _close(O, ref.numpy(), 1e-13, f"window {W} torch sdpa O")
    O, L = A.attention_ref(q, k, v, True, scale, window=1)
    diag = np.arange(Sq) + (Skv - Sq)
    g = Hq // Hkv
    for h in range(Hq):
        _close(O[:, h], v[:, h // g, diag], 1e-14, "window 1 O")
        _close(L[:, h], scale * np.einsum("bid,bid->bi", q[:, h], k[:, h // g, diag]), 1e-14,
               "window 1 LSE")
    Oc, Lc = A.attention_ref(q, k, v, True, scale)
    for W in (Skv, Skv + 5):
        O, L = A.attention_ref(q, k, v, True, scale, window=W)
        assert np.array_equal(O, Oc) and np.array_equal(L, Lc), "window >= Skv is causal"


def pin_fwd_bias(A):
    """Additive mask C given as a tensor: torch float64 sdpa with the same
    float mask (alone and with the causal pattern), 50-digit brute force
    with -inf entries, a constant per row (O unchanged, LSE shifted by it),
    the causal pattern written as a 0 / -inf bias, broadcast batch / head
    dimensions, and a row with every key masked (O = 0, LSE = -inf)."""
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 9, 14, 8
    q = _rand(70, B, Hq, Sq, d)
    k = _rand(71, B, Hkv, Skv, d)
    v = _rand(72, B, Hkv, Skv, d)
    bias = _rand(73, B, Hq, Sq, Skv, mult=2.0)
    scale = 1 / math.sqrt(d)
    kt = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vt = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    causal_c = np.where(np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq), 0.0,
                        -math.inf)
    for causal in (False, True):
        O, L = A.attention_ref(q, k, v, causal, scale, bias=bias)
        mask = torch.from_numpy(bias + (causal_c if causal else 0.0))
        ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q), kt, vt,
                                                               attn_mask=mask, scale=scale)
        _close(O, ref.numpy(), 1e-13, f"bias sdpa O causal={causal}")
    # brute force, -inf entries included
    bq, bk, bv = q[:1, :2, :4, :3], k[:1, :1, :6, :3], v[:1, :1, :6, :3]
    bb = bias[:1, :2, :4, :6].copy()
    bb[0, 0, 1, 2] = bb[0, 1, 3, 0] = -math.inf
    O, L = A.attention_ref(bq, bk, bv, False, 0.5, bias=bb)
    mpmath.mp.dps = 50
    for h in range(2):
        for i in range(4):
            es = [mpmath.mpf(0) if bb[0, h, i, j] == -math.inf else mpmath.exp(
                mpmath.mpf(0.5) * mpmath.fsum(mpmath.mpf(bq[0, h, i, c]) * mpmath.mpf(bk[0, 0, j, c])
                                              for c in range(3)) + mpmath.mpf(bb[0, h, i, j]))
                  for j in range(6)]
            den = mpmath.fsum(es)
            for c in range(3):
                _close(O[0, h, i, c], float(mpmath.fsum(e * mpmath.mpf(bv[0, 0, j, c])
                                                         for j, e in enumerate(es)) / den),
                       1e-13, "bias mpmath O")
            _close(L[0, h, i], float(mpmath.log(den)), 1e-13, "bias mpmath LSE")
    # a constant per row: softmax shift invariance
    cst = _rand(74, B, Hq, Sq, 1, mult=5.0)
    O0, L0 = A.attention_ref(q, k, v, True, scale)
    O1, L1 = A.attention_ref(q, k, v, True, scale, bias=np.broadcast_to(cst, (B, Hq, Sq, Skv)))
    _close(O1, O0, 1e-13, "constant bias O")
    _close(L1, L0 + cst[..., 0], 1e-13, "constant bias LSE")
    # the causal pattern as a bias; broadcast dimensions
    Oc, Lc = A.attention_ref(q, k, v, False, scale,
                             bias=np.broadcast_to(causal_c, (B, Hq, Sq, Skv)))
    _close(Oc, O0, 1e-14, "causal as bias O")
    _close(Lc, L0, 1e-14, "causal as bias LSE")
    shared = bias[:1, :1]
    Ob, Lb = A.attention_ref(q, k, v, True, scale, bias=np.broadcast_to(shared, bias.shape))
    Oe, Le = A.attention_ref(q, k, v, True, scale, bias=np.repeat(np.repeat(shared, B, 0), Hq, 1))
    assert np.array_equal(Ob, Oe) and np.array_equal(Lb, Le), "broadcast bias"
    # a row with every key masked
    dead = bias.copy()
    dead[1, 2, 5, :] = -math.inf
    O, L = A.attention_ref(q, k, v, False, scale, bias=dead)
    assert np.all(O[1, 2, 5] == 0) and L[1, 2, 5] == -math.inf, "fully masked row"
    Or, Lr = A.attention_ref(q, k, v, False, scale, bias=bias)
    keep = np.ones((B, Hq, Sq), dtype=bool)
    keep[1, 2, 5] = False
    _close(O[keep], Or[keep], 0.0, "other rows unchanged")


def pin_fwd_invariants(A):
    """Key shift moves LSE by scale q.u and keeps O; joint (K, V) row
    permutation keeps O (non-causal); grouped heads equal repeated heads."""
    B, Hq, Hkv, Sq, Skv, d = 1, 4, 2, 5, 8, 6
    q = _rand(17, B, Hq, Sq, d)
    k = _rand(18, B, Hkv, Skv, d)
    v = _rand(19, B, Hkv, Skv, d)
    u = _rand(20, d)
    scale = 0.4
    for causal in (False, True):
        O, L = A.attention_ref(q, k, v, causal, scale)
        O2, L2 = A.attention_ref(q, k + u, v, causal, scale)
        _close(O2, O, 1e-13, "shift O")
        _close(L2, L + scale * (q @ u), 1e-13, "shift LSE")
        rep = Hq // Hkv
        O3, L3 = A.attention_ref(q, np.repeat(k, rep, axis=1), np.repeat(v, rep, axis=1), causal, scale)
        _close(O3, O, 0.0, "GQA = repeated heads O")
        _close(L3, L, 0.0, "GQA = repeated heads LSE")
    perm = _rng(21).permutation(Skv)
    O, L = A.attention_ref(q, k, v, False, scale)
    O4, L4 = A.attention_ref(q, k[:, :, perm], v[:, :, perm], False, scale)
    _close(O4, O, 1e-13, "permutation O")
    _close(L4, L, 1e-13, "permutation LSE")


# ---------------------------------------------------------------- monoid

def pin_monoid_golden(A):
    """Block states and their merge on the hand-worked example."""
    gd = _golden()
    mo = gd["monoid"]
    w = np.asarray(gd["w"], dtype=np.float64)
    s = np.log(w)[None, :]
    V = np.asarray(gd["V"], dtype=np.float64)
    b1 = A.block_state(s[:, :2], V[:2])
    b2 = A.block_state(s[:, 2:], V[2:])
    for st, ref, nm in [(b1, mo["block1"], "block1"), (b2, mo["block2"], "block2")]:
        _close(st[0], [math.log(_frac(ref["m_exp"]))], 1e-15, nm + " m")
        _close(st[1], [_frac(ref["l"])], 1e-15, nm + " l")
        _close(st[2], [[_frac(x) for x in ref["o"]]], 1e-15, nm + " o")
    mg = A.merge(b1, b2)
    _close(mg[0], [math.log(_frac(mo["merged"]["m_exp"]))], 1e-15, "merged m")
    _close(mg[1], [_frac(mo["merged"]["l"])], 1e-15, "merged l")
    _close(mg[2], [[_frac(x) for x in mo["merged"]["o"]]], 1e-15, "merged o")
    O, L = A.finalize(mg)
    _close(O, [[0.3, 1.1]], 1e-15, "merged O")
    _close(L, [math.log(10.0)], 1e-15, "merged LSE")


def pin_monoid_identity(A):
    """merge(e, x) = x = merge(x, e) exactly; merging two identities stays
    the identity without NaN."""
    n, dv = 5, 3
    s = _rand(22, n, 7)
    s[1, :] = -math.inf                     # a row with no allowed key
    x = A.block_state(s, _rand(23, 7, dv))
    e = A.identity_state(n, dv)
    for y in (A.merge(e, x), A.merge(x, e)):
        for a, b in zip(y, x):
            assert np.array_equal(a, b), "identity law broken"
    ee = A.merge(e, e)
    assert np.all(ee[0] == -math.inf) and np.all(ee[1] == 0) and np.all(ee[2] == 0)
    assert not np.any(np.isnan(ee[1])) and not np.any(np.isnan(ee[2]))


def pin_monoid_chunkings(A):
    """Any partition of the keys and any merge tree gives the unchunked
    result (associativity), also the recurrence in the page's own order."""
    B, Hq, Hkv, Sq, Skv, d = 1, 2, 1, 9, 29, 5
    q = _rand(24, B, Hq, Sq, d, mult=2.0)
    k = _rand(25, B, Hkv, Skv, d)
    v = _rand(26, B, Hkv, Skv, d)
    scale = 0.8
    rng = _rng(27)

    def random_tree(states):
        states = list(states)
        while len(states) > 1:
            i = int(rng.integers(0, len(states) - 1))
            states[i:i + 2] = [A.merge(states[i], states[i + 1])]
        return states[0]

    for causal in (False, True):
        O, L = A.attention_ref(q, k, v, causal, scale)
        for c in (1, 3, 4, 16, Skv):
            bnd = list(range(0, Skv, c)) + [Skv]
            for tree in (None, "pairwise", random_tree):
                Om, Lm = A.attention_monoid(q, k, v, causal, scale, bnd, tree)
                _close(Om, O, 1e-13, f"chunk {c} O")
                _close(Lm, L, 1e-13, f"chunk {c} LSE")
        for blk in (1, 3, 8, Skv):
            for h in range(Hq):
                s = A.scores(q, k, causal, scale, 0, h)
                Or, Lr = A.online_softmax_recurrence(s, v[0, 0], blk)
                _close(Or, O[0, h], 1e-13, f"recurrence {blk} O")
                _close(Lr, L[0, h], 1e-13, f"recurrence {blk} LSE")
    # Non-contiguous partitions: key tiles of tk keys dealt to n sets (tile t
    # to set t % n; some sets empty), the sets' states merged in a shuffled
    # order, give the unchunked result too (associativity and commutativity).
    for causal in (False, True):
        O, L = A.attention_ref(q, k, v, causal, scale)
        for h in range(Hq):
            s = A.scores(q, k, causal, scale, 0, h)
            for n, tk in ((3, 4), (5, 2), (16, 2), (7, 1)):
                sets = [[j for j in range(Skv) if (j // tk) % n == t] for t in range(n)]
                states = [A.block_state(s[:, idx], v[0, 0][idx]) for idx in sets]
                st = A.identity_state(Sq, d)
                for i in rng.permutation(n):
                    st = A.merge(st, states[i])
                Om, Lm = A.finalize(st)
                _close(Om, O[0, h], 1e-13, f"dealt tiles n={n} tk={tk} O")
                _close(Lm, L[0, h], 1e-13, f"dealt tiles n={n} tk={tk} LSE")
    # commutativity of merge on real states
    s = _rand(28, 4, 10)
    vv = _rand(29, 10, 3)
    x, y = A.block_state(s[:, :4], vv[:4]), A.block_state(s[:, 4:], vv[4:])
    for a, b in zip(A.merge(x, y), A.merge(y, x)):
        _close(a, b, 1e-15, "commutativity")


def pin_monoid_lse(A):
    """The LSE of a merge is the log-add-exp of the parts' LSEs."""
    s = _rand(30, 6, 12, mult=3.0)
    vv = _rand(31, 12, 2)
    x, y = A.block_state(s[:, :5], vv[:5]), A.block_state(s[:, 5:], vv[5:])
    _, lx = A.finalize(x)
    _, ly = A.finalize(y)
    _, lm = A.finalize(A.merge(x, y))
    _close(lm, np.logaddexp(lx, ly), 1e-14, "merged LSE")
    _close(lm, scipy.special.logsumexp(s, axis=1), 1e-14, "merged LSE vs scipy")


# ---------------------------------------------------------------- decode

def pin_decode(A):
    """Split-KV decode equals the unsplit single-row attention and the last
    row of a causal prefill over the same keys; every split's finalised
    partial is attention over that chunk alone."""
    B, Hq, Hkv, Skv, d = 2, 8, 2, 50, 8
    k = _rand(32, B, Hkv, Skv, d)
    v = _rand(33, B, Hkv, Skv, d)
    qfull = _rand(34, B, Hq, Skv, d)
    q = qfull[:, :, -1:, :]
    scale = 1 / math.sqrt(d)
    Oref, Lref = A.attention_ref(q, k, v, False, scale)
    Opre, Lpre = A.attention_ref(qfull, k, v, True, scale)
    for n in (1, 3, 7, 16, 64):
        O, L = A.decode_ref(q, k, v, scale, n)
        _close(O, Oref, 1e-13, f"decode n={n} O")
        _close(L, Lref, 1e-13, f"decode n={n} LSE")
        _close(O[:, :, 0], Opre[:, :, -1], 1e-13, "decode = last causal row")
        _close(L[:, :, 0], Lpre[:, :, -1], 1e-13, "decode LSE = last causal row")
        bnd = A.split_bounds(Skv, n)
        assert bnd[0] == 0 and bnd[-1] == Skv and len(bnd) == n + 1
        c = -(-Skv // n)
        assert all(0 <= bnd[i + 1] - bnd[i] <= c for i in range(n))
        assert all(bnd[i + 1] - bnd[i] == c for i in range(Skv // c))
        m, l, acc = A.decode_partials(q, k, v, scale, n)
        for sp in range(n):
            a, z = bnd[sp], bnd[sp + 1]
            if z == a:
                assert np.all(m[sp] == -math.inf) and np.all(l[sp] == 0)
                continue
            Oc, Lc = A.attention_ref(q, k[:, :, a:z], v[:, :, a:z], False, scale)
            _close(acc[sp] / l[sp][..., None], Oc[:, :, 0], 1e-13, "split partial O")
            _close(m[sp] + np.log(l[sp]), Lc[:, :, 0], 1e-13, "split partial LSE")


def pin_decode_paged(A):
    """Paged decode equals plain attention of each stream's query over its
    first seq_len keys, written out contiguously: an identity block table,
    a shuffled page pool, ragged, empty, negative and over-capacity lengths,
    and page ids outside the pool (pages of zeros)."""
    B, Hq, Hkv, S, d, ps = 3, 4, 2, 40, 6, 8
    npg = S // ps
    k = _rand(60, B, Hkv, S, d)
    v = _rand(61, B, Hkv, S, d)
    q = _rand(62, B, Hq, 1, d, mult=2.0)
    scale = 0.4
    rng = _rng(63)

    def pool(x):  # page b * npg + i holds rows [i ps, (i + 1) ps) of stream b
        return x.reshape(B, Hkv, npg, ps, d).transpose(0, 2, 1, 3, 4).reshape(B * npg, Hkv, ps, d)

    def plain(kk, vv, lens):
        O = np.zeros((B, Hq, 1, d))
        L = np.full((B, Hq, 1), -math.inf)
        for b in range(B):
            n = int(min(max(lens[b], 0), S))
            if n:
                O[b:b + 1], L[b:b + 1] = A.attention_ref(q[b:b + 1], kk[b:b + 1, :, :n],
                                                         vv[b:b + 1, :, :n], False, scale)
        return O, L

    kp, vp = pool(k), pool(v)
    table = np.arange(B * npg).reshape(B, npg)
    for lens in ([S, 17, 1], [8, 9, 33], [0, S + 100, -5]):
        lens = np.array(lens)
        O, L = A.decode_paged_ref(q, kp, vp, table, lens, scale)
        Or, Lr = plain(k, v, lens)
        _close(O, Or, 1e-14, f"paged O lens={lens.tolist()}")
        assert np.array_equal(np.isinf(L), np.isinf(Lr)), "empty streams"
        _close(np.where(np.isinf(L), 0, L), np.where(np.isinf(Lr), 0, Lr), 1e-14, "paged LSE")
        # the same pages at shuffled places in the pool
        perm = rng.permutation(B * npg)
        kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
        kp2[perm], vp2[perm] = kp, vp
        O2, L2 = A.decode_paged_ref(q, kp2, vp2, perm[table], lens, scale)
        assert np.array_equal(O2, O) and np.array_equal(L2, L), "shuffled pool"
    # full lengths: the split-KV decode of the contiguous cache
    Od, Ld = A.decode_ref(q, k, v, scale, 5)
    O, L = A.decode_paged_ref(q, kp, vp, table, np.full(B, S), scale)
    _close(O, Od, 1e-13, "paged vs split decode O")
    _close(L, Ld, 1e-13, "paged vs split decode LSE")
    # page ids outside the pool read as zeros
    bad = table.copy()
    bad[0, 1], bad[1, 4] = -1, B * npg
    kz, vz = k.copy(), v.copy()
    kz[0, :, ps:2 * ps] = 0
    vz[0, :, ps:2 * ps] = 0
    kz[1, :, 4 * ps:5 * ps] = 0
    vz[1, :, 4 * ps:5 * ps] = 0
    O, L = A.decode_paged_ref(q, kp, vp, bad, np.full(B, S), scale)
    Or, Lr = plain(kz, vz, np.full(B, S))
    _close(O, Or, 1e-14, "invalid page ids O")
    _close(L, Lr, 1e-14, "invalid page ids LSE")


# ---------------------------------------------------------------- backward

def _loss_grad_fd(A, q, k, v, do, causal, scale, eps=1e-6):
    """Central finite differences of L = sum(dO * O) w.r.t. q, k, v."""
    grads = []
    for which in range(3):
        base = [q, k, v]
        x = base[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xp[idx] += eps
            xm = x.copy()
            xm[idx] -= eps
            args_p = list(base)
            args_p[which] = xp
            args_m = list(base)
            args_m[which] = xm
            Op, _ = A.attention_ref(*args_p, causal, scale)
            Om, _ = A.attention_ref(*args_m, causal, scale)
            g[idx] = (np.sum(do * Op) - np.sum(do * Om)) / (2 * eps)
        grads.append(g)
    return grads


def pin_bwd_finite_difference(A):
    for seed, (B, Hq, Hkv, Sq, Skv, d), causal in [
        (40, (1, 2, 1, 3, 4, 3), True),
        (41, (1, 2, 2, 3, 3, 2), False),
    ]:
        q = _rand(seed, B, Hq, Sq, d)
        k = _rand(seed + 1, B, Hkv, Skv, d)
        v = _rand(seed + 2, B, Hkv, Skv, d)
        do = _rand(seed + 3, B, Hq, Sq, d)
        dq, dk, dv, _ = A.attention_bwd_ref(q, k, v, do, causal, 0.6)
        fq, fk, fv = _loss_grad_fd(A, q, k, v, do, causal, 0.6)
        _close(dq, fq, 1e-7, "fd dQ")
        _close(dk, fk, 1e-7, "fd dK")
        _close(dv, fv, 1e-7, "fd dV")


def pin_bwd_autograd(A):
    """torch.autograd in float64 on an explicit-softmax formula."""
    B, Hq, Hkv, Sq, Skv, d = 2, 4, 2, 7, 12, 8
    q = _rand(42, B, Hq, Sq, d)
    k = _rand(43, B, Hkv, Skv, d)
    v = _rand(44, B, Hkv, Skv, d)
    do = _rand(45, B, Hq, Sq, d)
    scale = 1 / math.sqrt(d)
    for causal in (False, True):
        qt = torch.from_numpy(q).requires_grad_()
        kt = torch.from_numpy(k).requires_grad_()
        vt = torch.from_numpy(v).requires_grad_()
        kr = kt.repeat_interleave(Hq // Hkv, dim=1)
        vr = vt.repeat_interleave(Hq // Hkv, dim=1)
        s = (qt @ kr.transpose(-1, -2)) * scale
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Skv)[None, :]
            s = s.masked_fill(j > i + (Skv - Sq), float("-inf"))
        o = torch.softmax(s, dim=-1) @ vr
        o.backward(torch.from_numpy(do))
        dq, dk, dv, D = A.attention_bwd_ref(q, k, v, do, causal, scale)
        _close(dq, qt.grad.numpy(), 1e-12, "autograd dQ")
        _close(dk, kt.grad.numpy(), 1e-12, "autograd dK")
        _close(dv, vt.grad.numpy(), 1e-12, "autograd dV")
        _close(D, np.sum(do * o.detach().numpy(), axis=-1), 1e-12, "D = rowsum(dO*O)")
    # an additive bias tensor (with some -inf entries), with and without causal
    bias = _rand(46, B, Hq, Sq, Skv, mult=1.5)
    bias[0, 1, 3, :4] = -math.inf
    for causal in (False, True):
        qt = torch.from_numpy(q).requires_grad_()
        kt = torch.from_numpy(k).requires_grad_()
        vt = torch.from_numpy(v).requires_grad_()
        kr = kt.repeat_interleave(Hq // Hkv, dim=1)
        vr = vt.repeat_interleave(Hq // Hkv, dim=1)
        s = (qt @ kr.transpose(-1, -2)) * scale + torch.from_numpy(bias)
        if causal:
            i = torch.arange(Sq)[:, None]
            j = torch.arange(Skv)[None, :]
            s = s.masked_fill(j > i + (Skv - Sq), float("-inf"))
        o = torch.softmax(s, dim=-1) @ vr
        o.backward(torch.from_numpy(do))
        dq, dk, dv, D = A.attention_bwd_ref(q, k, v, do, causal, scale, bias=bias)
        _close(dq, qt.grad.numpy(), 1e-12, f"bias autograd dQ causal={causal}")
        _close(dk, kt.grad.numpy(), 1e-12, f"bias autograd dK causal={causal}")
        _close(dv, vt.grad.numpy(), 1e-12, f"bias autograd dV causal={causal}")
    # sliding windows (causal)
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Skv)[None, :]
    for W in (1, 3, 8):
        qt = torch.from_numpy(q).requires_grad_()
        kt = torch.from_numpy(k).requires_grad_()
        vt = torch.from_numpy(v).requires_grad_()
        kr = kt.repeat_interleave(Hq // Hkv, dim=1)
        vr = vt.repeat_interleave(Hq // Hkv, dim=1)
        s = (qt @ kr.transpose(-1, -2)) * scale
        keep = (j <= i + (Skv - Sq)) & (j > i + (Skv - Sq) - W)
        s = s.masked_fill(~keep, float("-inf"))
        o = torch.softmax(s, dim=-1) @ vr
        o.backward(torch.from_numpy(do))
        dq, dk, dv, D = A.attention_bwd_ref(q, k, v, do, True, scale, window=W)
        _close(dq, qt.grad.numpy(), 1e-12, f"window {W} autograd dQ")
        _close(dk, kt.grad.numpy(), 1e-12, f"window {W} autograd dK")
        _close(dv, vt.grad.numpy(), 1e-12, f"window {W} autograd dV")


def pin_bwd_golden(A):
    """The hand-worked backward example."""
    gd = _golden()["backward"]
    q, k, v = _golden_qkv(gd["w"], gd["V"])
    q = q[:, :, :1]
    do = np.asarray(gd["dO"], dtype=np.float64)[None, None, None]
    dq, dk, dv, D = A.attention_bwd_ref(q, k, v, do, False, 0.5)
    _close(D[0, 0], [_frac(gd["D"])], 1e-15, "golden D")
    _close(dv[0, 0], [[_frac(x) for x in r] for r in gd["dV"]], 1e-15, "golden dV")
    _close(dk[0, 0], [[_frac(x) for x in r] for r in gd["dK"]], 1e-15, "golden dK")
    _close(dq[0, 0, 0], [_frac(x) * math.log(3.0) for x in gd["dQ_over_ln3"]], 1e-15, "golden dQ")


def pin_bwd_identities(A):
    """sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i per key/value head; equal
    key rows give dQ = 0; Q = 0 gives dV_j = sum over rows seeing j of
    dO_i / (number of keys row i sees)."""
    B, Hq, Hkv, Sq, Skv, d = 1, 4, 2, 6, 9, 5
    q = _rand(46, B, Hq, Sq, d)
    k = _rand(47, B, Hkv, Skv, d)
    v = _rand(48, B, Hkv, Skv, d)
    do = _rand(49, B, Hq, Sq, d)
    g = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv, _ = A.attention_bwd_ref(q, k, v, do, causal, 0.5)
        _close(dk.sum(axis=2), np.zeros((B, Hkv, d)), 1e-13, "sum dK")
        _close(dv.sum(axis=2), do.reshape(B, Hkv, g, Sq, d).sum(axis=(2, 3)), 1e-13, "sum dV")
        keq = np.broadcast_to(k[:, :, :1], k.shape).copy()
        dq0, _, _, _ = A.attention_bwd_ref(q, keq, v, do, causal, 0.5)
        _close(dq0, np.zeros_like(dq0), 1e-14, "equal keys dQ")
        _, _, dvz, _ = A.attention_bwd_ref(np.zeros_like(q), k, v, do, causal, 0.5)
        ref = np.zeros_like(v)
        for h in range(Hq):
            for i in range(Sq):
                n = _allowed(i, Sq, Skv, causal)
                ref[0, h // g, :n] += do[0, h, i] / n
        _close(dvz, ref, 1e-14, "Q=0 dV")


FORWARD_PINS = [pin_fwd_mpmath, pin_fwd_golden, pin_fwd_uniform, pin_fwd_onehot,
                pin_fwd_single_key, pin_fwd_scipy, pin_fwd_torch_sdpa, pin_fwd_window,
                pin_fwd_bias, pin_fwd_invariants]
MONOID_PINS = [pin_monoid_golden, pin_monoid_identity, pin_monoid_chunkings, pin_monoid_lse]
DECODE_PINS = [pin_decode, pin_decode_paged]
BACKWARD_PINS = [pin_bwd_finite_difference, pin_bwd_autograd, pin_bwd_golden, pin_bwd_identities]
ALL_PINS = FORWARD_PINS + MONOID_PINS + DECODE_PINS + BACKWARD_PINS
