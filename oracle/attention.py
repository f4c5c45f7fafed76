"""Float64 CPU oracle for online-softmax attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

Every function here is written from the text of the pages, not from any
kernel.  Citations name the page title and the section or equation:

* "Compilers and Kernels", section "FlashAttention changes the algorithm
  around IO": the first display equation (the definition of scaled
  dot-product attention with additive mask C and row statistics m_i, l_i),
  its "where" list (C in (R u {-inf})^{NxN}, every query row keeps at least
  one allowed key), the second display equation (the blockwise recurrence
  b_t, m_t, alpha_t, l_t, o_t from m_0=-inf, l_0=0, o_0=0) and the closing
  equation O_i = o_T / l_T.
* "Tang, a compiler that derives GPU kernels and bounds how fast they can
  run", Abstract: online softmax recognised as a monoid; gradients of
  comprehensions are comprehensions, so the backward exists and writes no
  intermediates.
* "Don't Write Kernels, Derive Them", section "What happened": logsumexp is
  one of the operations that emerge.

Readings where the pages are silent (each is also listed in the design notes):

* causal alignment for Sq != Skv is bottom-right: key j is allowed for query
  i iff j <= i + (Skv - Sq); causal with Sq > Skv would leave a row with no
  allowed key, which the definition excludes;
* an additive bias is the mask C itself, given as a tensor: C[b, h, i, j]
  (any real or -inf) is added to the scaled scores, on top of the causal and
  window patterns; a row whose every key is -inf has O = 0 and LSE = -inf
  (the definition asks for at least one allowed key per row);
* a sliding window of W keys (W > 0, causal only) is one more pattern of the
  additive mask C: key j is allowed for query i iff
  i + (Skv - Sq) - W < j <= i + (Skv - Sq), so every row keeps its diagonal
  key; W <= 0 means no window;
* grouped-query heads: query head h reads key/value head h // (Hq // Hkv);
* LSE is the natural-log log-sum-exp of the scaled, masked scores, m + ln l;
* the scale multiplies the exact dot product;
* merging with the identity (m = -inf) is exact: its weight is 0, never
  exp(-inf - -inf);
* split-KV boundaries are contiguous chunks of ceil(Skv / n_splits) keys, the
  last one possibly shorter (or empty), partials left unnormalised;
* paged decode: the key/value pools are [n_pages, Hkv, page_size, d]; key t
  of stream b is row t % page_size of page block_table[b, t // page_size];
  the stream's length is clamped to [0, max_pages * page_size]; a page id
  outside [0, n_pages) stands for a page of zeros; a stream with no keys
  has O = 0 and LSE = -inf (the definition needs at least one allowed key);
* the backward is the plain derivative of the definition, with P recomputed
  from the saved LSE: dV = P^T dO, dP = dO V^T, D_i = sum_j P_ij dP_ij,
  dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q, grouped heads summing
  into their shared key/value head, masked pairs contributing zero.

All arrays are numpy float64 in [B, H, S, d] order.  Callers pass the exact
values the GPU sees (bf16 inputs upcast exactly to float64).
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -math.inf

# Rows per block when forming explicit score rows; bounds memory to
# block * Skv float64 values, it does not change what is computed.
_ROW_BLOCK = 512


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, d]")
    B, Hq, Sq, d = q.shape
    Bk, Hkv, Skv, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3] or v.shape[0] != B:
        raise ValueError("shape mismatch between q, k, v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Sq, Skv, d, v.shape[3]


def mask_matrix(rows, Sq, Skv, causal, window=0):
    """Additive mask C restricted to the given query rows: 0 or -inf.  With
    window W > 0 (causal only), keys more than W - 1 before the diagonal are
    masked too."""
    if window > 0 and not causal:
        raise ValueError("a sliding window needs the causal mask")
    rows = np.asarray(rows)
    c = np.zeros((rows.size, Skv))
    if causal:
        j = np.arange(Skv)[None, :]
        c[j > rows[:, None] + (Skv - Sq)] = NEG_INF
        if window > 0:
            c[j <= rows[:, None] + (Skv - Sq) - window] = NEG_INF
    return c


def scores(q, k, causal, scale, b, hq, rows=None, window=0, bias=None):
    """S = Q K^T * scale + C for one (batch, query head), selected rows.
    bias: optional [B, Hq, Sq, Skv] additive part of C (broadcast views of a
    smaller array are fine)."""
    B, Hq, Sq, d = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    g = Hq // Hkv
    if rows is None:
        rows = np.arange(Sq)
    s = (q[b, hq][rows] @ k[b, hq // g].T) * scale
    if bias is not None:
        s = s + bias[b, hq][rows]
    return s + mask_matrix(rows, Sq, Skv, causal, window)


def attention_ref(q, k, v, causal, scale, rows=None, window=0, bias=None):
    """Scaled dot-product attention, the plain definition.

    Follows the first display equation of "Compilers and Kernels", section
    "FlashAttention changes the algorithm around IO": m_i = max_j S_ij,
    l_i = sum_j exp(S_ij - m_i), P_ij = exp(S_ij - m_i) / l_i, O = P V;
    LSE_i = m_i + ln l_i (logsumexp, "Don't Write Kernels, Derive Them").

    rows: optional sorted array of query-row indices; when given, only those
    rows are computed and O is [B, Hq, len(rows), dv], LSE [B, Hq, len(rows)].
    window: sliding-window width W (causal only; <= 0: none).
    bias: optional additive mask values [B, Hq, Sq, Skv] (may hold -inf).
    Returns (O, LSE); a row with no allowed key gets O = 0, LSE = -inf.
    """
    B, Hq, Hkv, Sq, Skv, d, dv = _check_shapes(q, k, v)
    if causal and Sq > Skv:
        raise ValueError("causal with Sq > Skv leaves a query row with no allowed key")
    g = Hq // Hkv
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.empty((B, Hq, rows.size, dv))
    lse = np.empty((B, Hq, rows.size))
    for b in range(B):
        for h in range(Hq):
            vv = v[b, h // g]
            for r0 in range(0, rows.size, _ROW_BLOCK):
                rr = rows[r0:r0 + _ROW_BLOCK]
                s = scores(q, k, causal, scale, b, h, rr, window, bias)
                m = s.max(axis=1)
                live = m != NEG_INF
                e = np.zeros_like(s)
                e[live] = np.exp(s[live] - m[live][:, None])
                l = e.sum(axis=1)
                o = np.zeros((rr.size, dv))
                o[live] = (e[live] @ vv) / l[live][:, None]
                out[b, h, r0:r0 + rr.size] = o
                lse[b, h, r0:r0 + rr.size] = np.where(live, m + np.log(np.where(live, l, 1.0)),
                                                      NEG_INF)
    return out, lse


# ---------------------------------------------------------------------------
# The online-softmax monoid.
#
# A state is a triple (m, l, o) per query row: running maximum, running
# normaliser and accumulator rescaled to exp(-m).  The identity is
# (-inf, 0, 0), the initial state of the blockwise recurrence.  Arrays:
# m [n], l [n], o [n, dv].
# ---------------------------------------------------------------------------

def identity_state(n, dv):
    """(m_0, l_0, o_0) = (-inf, 0, 0): the recurrence's initial state."""
    return np.full(n, NEG_INF), np.zeros(n), np.zeros((n, dv))


def _weight(m_from, m_to):
    """exp(m_from - m_to), exactly 0 when m_from is -inf (identity element)."""
    w = np.zeros_like(m_from)
    live = m_from != NEG_INF
    w[live] = np.exp(m_from[live] - m_to[live])
    return w


def block_state(s, v):
    """State of one key block on its own: (b, sum exp(s - b), sum exp(s - b) v).

    s: [n, nb] scores with -inf for disallowed keys; v: [nb, dv].  A row with
    no allowed key in the block yields the identity for that row.
    """
    n = s.shape[0]
    m, l, o = identity_state(n, v.shape[1])
    if s.shape[1] == 0:
        return m, l, o
    b = s.max(axis=1)
    live = b != NEG_INF
    e = np.zeros_like(s)
    e[live] = np.exp(s[live] - b[live][:, None])
    m[live] = b[live]
    l[:] = e.sum(axis=1)
    o[:] = e @ v
    return m, l, o


def merge(x, y):
    """Monoid operation: rescale both states to the common maximum and add.

    m = max(m_x, m_y); l = w_x l_x + w_y l_y; o = w_x o_x + w_y o_y with
    w = exp(m_. - m).  The blockwise recurrence of "Compilers and Kernels"
    (second display equation) is the special case where y is one block's
    state; the general two-sided form is what lets independent key splits
    be combined in any grouping.
    """
    mx, lx, ox = x
    my, ly, oy = y
    m = np.maximum(mx, my)
    wx = _weight(mx, m)
    wy = _weight(my, m)
    return m, wx * lx + wy * ly, wx[:, None] * ox + wy[:, None] * oy


def finalize(state):
    """O_i = o_T / l_T (closing equation) and LSE_i = m_T + ln l_T."""
    m, l, o = state
    return o / l[:, None], m + np.log(l)


def online_softmax_recurrence(s, v, block):
    """The blockwise recurrence of "Compilers and Kernels", second display
    equation, in its own order and notation, for one head.

    s: [n, N] masked scores, v: [N, dv], block: keys per block.  For each
    block B_t: b_t = max_j S_ij, m_t = max(m_{t-1}, b_t),
    alpha_t = exp(m_{t-1} - m_t), l_t = alpha_t l_{t-1} + sum exp(S_ij - m_t),
    o_t = alpha_t o_{t-1} + sum exp(S_ij - m_t) v_j.  Returns (O, LSE).
    alpha_t is taken as 0 while m_{t-1} = -inf (no key seen yet).
    """
    n, N = s.shape
    m, l, o = identity_state(n, v.shape[1])
    for j0 in range(0, N, block):
        sb = s[:, j0:j0 + block]
        vb = v[j0:j0 + block]
        b_t = sb.max(axis=1)
        m_t = np.maximum(m, b_t)
        alpha = _weight(m, m_t)
        e = np.zeros_like(sb)
        live = m_t != NEG_INF
        e[live] = np.exp(sb[live] - m_t[live][:, None])
        l = alpha * l + e.sum(axis=1)
        o = alpha[:, None] * o + e @ vb
        m = m_t
    return o / l[:, None], m + np.log(l)


def attention_monoid(q, k, v, causal, scale, boundaries, tree=None, window=0):
    """Attention as a fold of key-block states under `merge`.

    boundaries: increasing key offsets starting at 0 and ending at Skv that
    partition the keys into blocks.  tree: None folds left to right; "pairwise"
    merges neighbours level by level; a callable receives the list of block
    states and must return one state (any grouping is allowed for a monoid).
    Returns (O, LSE).
    """
    B, Hq, Hkv, Sq, Skv, d, dv = _check_shapes(q, k, v)
    if boundaries[0] != 0 or boundaries[-1] != Skv:
        raise ValueError("boundaries must start at 0 and end at Skv")
    g = Hq // Hkv
    out = np.empty((B, Hq, Sq, dv))
    lse = np.empty((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            s = scores(q, k, causal, scale, b, h, window=window)
            vv = v[b, h // g]
            states = [block_state(s[:, a:z], vv[a:z])
                      for a, z in zip(boundaries[:-1], boundaries[1:])]
            if tree is None:
                acc = identity_state(Sq, dv)
                for st in states:
                    acc = merge(acc, st)
            elif tree == "pairwise":
                while len(states) > 1:
                    nxt = [merge(states[i], states[i + 1])
                           for i in range(0, len(states) - 1, 2)]
                    if len(states) % 2:
                        nxt.append(states[-1])
                    states = nxt
                acc = states[0]
            else:
                acc = tree(states)
            out[b, h], lse[b, h] = finalize(acc)
    return out, lse


# ---------------------------------------------------------------------------
# Split-KV decode: one query row per (batch, query head), all cached keys
# visible, keys cut into n_splits contiguous chunks whose unnormalised states
# are combined by the monoid.
# ---------------------------------------------------------------------------

def split_bounds(Skv, n_splits):
    """Contiguous chunk boundaries of ceil(Skv / n_splits) keys; trailing
    chunks may be short or empty."""
    c = -(-Skv // n_splits)
    return [min(s * c, Skv) for s in range(n_splits + 1)]


def decode_partials(q, k, v, scale, n_splits):
    """Per-split states for single-token decode.

    q: [B, Hq, 1, d]; k, v: [B, Hkv, Skv, d].  Returns (m, l, acc) with
    m, l: [n_splits, B, Hq] and acc: [n_splits, B, Hq, dv], each split's
    (b, sum exp(s - b), sum exp(s - b) v) over its own keys.
    """
    B, Hq, Hkv, Sq, Skv, d, dv = _check_shapes(q, k, v)
    if Sq != 1:
        raise ValueError("decode takes one query row per head")
    g = Hq // Hkv
    bounds = split_bounds(Skv, n_splits)
    m = np.empty((n_splits, B, Hq))
    l = np.empty((n_splits, B, Hq))
    acc = np.empty((n_splits, B, Hq, dv))
    for b in range(B):
        for h in range(Hq):
            s = (q[b, h] @ k[b, h // g].T) * scale  # [1, Skv]
            for sp in range(n_splits):
                a, z = bounds[sp], bounds[sp + 1]
                st = block_state(s[:, a:z], v[b, h // g][a:z])
                m[sp, b, h], l[sp, b, h], acc[sp, b, h] = st[0][0], st[1][0], st[2][0]
    return m, l, acc


def decode_combine(m, l, acc):
    """Fold the per-split states with `merge`, then finalise.

    Returns O [B, Hq, 1, dv] and LSE [B, Hq, 1].
    """
    n_splits, B, Hq = m.shape
    dv = acc.shape[-1]
    st = identity_state(B * Hq, dv)
    for sp in range(n_splits):
        st = merge(st, (m[sp].reshape(-1), l[sp].reshape(-1), acc[sp].reshape(-1, dv)))
    o, lse = finalize(st)
    return o.reshape(B, Hq, 1, dv), lse.reshape(B, Hq, 1)


def decode_ref(q, k, v, scale, n_splits):
    """Split-KV decode: partial states per chunk, combined by the monoid."""
    return decode_combine(*decode_partials(q, k, v, scale, n_splits))


# ---------------------------------------------------------------------------
# Paged, variable-length decode.  Paging changes only where the keys are
# stored: the result is attention of each stream's query row over that
# stream's keys in order ("Compilers and Kernels", FlashAttention section,
# first display equation), with all of its keys visible.
# ---------------------------------------------------------------------------

def paged_gather(pages, block_table, b, seq_len):
    """Keys (or values) 0 .. L-1 of stream b as a contiguous [Hkv, L, d]
    array.  pages: [n_pages, Hkv, page_size, d]; block_table: [B, max_pages]
    integers; L = seq_len clamped to [0, max_pages * page_size].  Key t is
    row t % page_size of page block_table[b, t // page_size]; a page id
    outside [0, n_pages) stands for a page of zeros."""
    n_pages, Hkv, ps, d = pages.shape
    L = min(max(int(seq_len), 0), block_table.shape[1] * ps)
    t = np.arange(L)
    pid = np.asarray(block_table[b])[t // ps].astype(np.int64)
    ok = (pid >= 0) & (pid < n_pages)
    out = np.zeros((L, Hkv, d))
    out[ok] = pages[pid[ok], :, (t % ps)[ok], :]
    return out.transpose(1, 0, 2)


def decode_paged_ref(q, k_pages, v_pages, block_table, seq_lens, scale):
    """Paged decode.  q: [B, Hq, 1, d]; k_pages, v_pages: [n_pages, Hkv,
    page_size, d]; block_table: [B, max_pages]; seq_lens: [B].  Returns
    O [B, Hq, 1, dv] and LSE [B, Hq, 1]; a stream with no keys gets O = 0
    and LSE = -inf."""
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query row per head")
    dv = v_pages.shape[-1]
    O = np.zeros((B, Hq, 1, dv))
    LSE = np.full((B, Hq, 1), NEG_INF)
    for b in range(B):
        kb = paged_gather(k_pages, block_table, b, seq_lens[b])
        if kb.shape[1] == 0:
            continue
        vb = paged_gather(v_pages, block_table, b, seq_lens[b])
        o, lse = attention_ref(q[b:b + 1], kb[None], vb[None], False, scale)
        O[b], LSE[b] = o[0], lse[0]
    return O, LSE


# ---------------------------------------------------------------------------
# Backward: P recomputed from the saved LSE, nothing quadratic kept between
# query heads ("Compilers and Kernels", closing paragraph of the FlashAttention
# section: the backward recomputes local score and probability tiles).
# ---------------------------------------------------------------------------

def attention_bwd_ref(q, k, v, do, causal, scale, lse=None, window=0, bias=None):
    """Gradients of O = softmax(scale Q K^T + C) V with respect to Q, K, V.

    lse: [B, Hq, Sq] saved forward statistic; computed from the definition
    when None.  Returns (dQ, dK, dV, D) where D_i = sum_j P_ij dP_ij.
    """
    B, Hq, Hkv, Sq, Skv, d, dv = _check_shapes(q, k, v)
    if causal and Sq > Skv:
        raise ValueError("causal with Sq > Skv leaves a query row with no allowed key")
    g = Hq // Hkv
    if lse is None:
        _, lse = attention_ref(q, k, v, causal, scale, window=window, bias=bias)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dvv = np.zeros_like(v)
    dd = np.empty((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, h // g], v[b, h // g]
            s = scores(q, k, causal, scale, b, h, window=window, bias=bias)
            live = lse[b, h] != NEG_INF                 # rows with at least one allowed key
            p = np.zeros_like(s)
            p[live] = np.exp(s[live] - lse[b, h][live][:, None])   # masked pairs: exp(-inf) = 0
            dp = do[b, h] @ vv.T
            D = (p * dp).sum(axis=1)
            ds = p * (dp - D[:, None])
            dvv[b, h // g] += p.T @ do[b, h]
            dq[b, h] = scale * (ds @ kk)
            dk[b, h // g] += scale * (ds.T @ q[b, h])
            dd[b, h] = D
    return dq, dk, dvv, dd
