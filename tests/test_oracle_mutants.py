"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant rewrites one expression of oracle/attention.py (a dropped term,
a wrong sign or index, a transposed operand, a missing guard), executes the
result as a separate module and runs the pins against it.  Only the copy is
changed, on the CPU; the real oracle is untouched.
"""
import os
import types

import pytest

from tests import oracle_pins as P

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")

# (name, old text, new text, occurrence index to replace)
MUTANTS = [
    ("scores without scale", "s = (q[b, hq][rows] @ k[b, hq // g].T) * scale",
     "s = (q[b, hq][rows] @ k[b, hq // g].T)", 0),
    ("causal top-left aligned", "c[j > rows[:, None] + (Skv - Sq)] = NEG_INF",
     "c[j > rows[:, None]] = NEG_INF", 0),
    ("causal drops diagonal", "c[j > rows[:, None] + (Skv - Sq)] = NEG_INF",
     "c[j >= rows[:, None] + (Skv - Sq)] = NEG_INF", 0),
    ("GQA key head modulo", "k[b, hq // g].T", "k[b, hq % Hkv].T", 0),
    ("GQA value head modulo", "vv = v[b, h // g]\n            for r0",
     "vv = v[b, h % Hkv]\n            for r0", 0),
    ("LSE without max", "np.where(live, m + np.log(np.where(live, l, 1.0)),",
     "np.where(live, np.log(np.where(live, l, 1.0)),", 0),
    ("O not normalised", "o[live] = (e[live] @ vv) / l[live][:, None]",
     "o[live] = (e[live] @ vv)", 0),
    ("O from keys", "o[live] = (e[live] @ vv) / l[live][:, None]",
     "o[live] = (e[live] @ k[b, h // g]) / l[live][:, None]", 0),
    ("merge weight sign", "w[live] = np.exp(m_from[live] - m_to[live])",
     "w[live] = np.exp(m_to[live] - m_from[live])", 0),
    ("merge drops a weight", "return m, wx * lx + wy * ly,", "return m, wx * lx + ly,", 0),
    ("identity unguarded", "live = m_from != NEG_INF", "live = np.ones_like(m_from, dtype=bool)", 0),
    ("finalize LSE sign", "return o / l[:, None], m + np.log(l)",
     "return o / l[:, None], m - np.log(l)", 0),
    ("block state unshifted", "e[live] = np.exp(s[live] - b[live][:, None])",
     "e[live] = np.exp(s[live])", 0),
    ("recurrence drops alpha", "l = alpha * l + e.sum(axis=1)", "l = l + e.sum(axis=1)", 0),
    ("split chunk floor", "c = -(-Skv // n_splits)", "c = max(Skv // n_splits, 1)", 0),
    ("decode without scale", "s = (q[b, h] @ k[b, h // g].T) * scale",
     "s = (q[b, h] @ k[b, h // g].T)", 0),
    ("window off by one", "c[j <= rows[:, None] + (Skv - Sq) - window] = NEG_INF",
     "c[j < rows[:, None] + (Skv - Sq) - window] = NEG_INF", 0),
    ("window ignored", "        if window > 0:\n            c[j <=",
     "        if window < 0:\n            c[j <=", 0),
    ("window top-left aligned", "c[j <= rows[:, None] + (Skv - Sq) - window] = NEG_INF",
     "c[j <= rows[:, None] - window] = NEG_INF", 0),
    ("paged row within page", "out[ok] = pages[pid[ok], :, (t % ps)[ok], :]",
     "out[ok] = pages[pid[ok], :, ((t + 1) % ps)[ok], :]", 0),
    ("paged page of next key", "pid = np.asarray(block_table[b])[t // ps]",
     "pid = np.asarray(block_table[b])[np.minimum((t + 1) // ps, block_table.shape[1] - 1)]", 0),
    ("paged length unclamped", "L = min(max(int(seq_len), 0), block_table.shape[1] * ps)",
     "L = max(int(seq_len), 0)", 0),
    ("paged invalid id wraps", "ok = (pid >= 0) & (pid < n_pages)",
     "pid = pid % n_pages\n    ok = pid >= 0", 0),
    ("paged empty stream NaN", "        if kb.shape[1] == 0:\n            continue",
     "        if kb.shape[1] == 0:\n            O[b] = np.nan\n            continue", 0),
    ("bwd dS sign", "ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])", 0),
    ("bwd dK without scale", "dk[b, h // g] += scale * (ds.T @ q[b, h])",
     "dk[b, h // g] += (ds.T @ q[b, h])", 0),
    ("bwd dV transposed", "dvv[b, h // g] += p.T @ do[b, h]",
     "dvv[b, h // g] += (p @ do[b, h]) if p.shape[0] == p.shape[1] else p.T @ do[b, h] * 0", 0),
    ("bwd dQ from values", "dq[b, h] = scale * (ds @ kk)", "dq[b, h] = scale * (ds @ vv)", 0),
    ("bwd D without P", "D = (p * dp).sum(axis=1)", "D = dp.sum(axis=1)", 0),
    ("bwd GQA overwrite", "dk[b, h // g] += scale", "dk[b, h // g] = scale", 0),
    ("bwd P without LSE", "p[live] = np.exp(s[live] - lse[b, h][live][:, None])",
     "p[live] = np.exp(s[live])", 0),
    ("bias dropped", "        s = s + bias[b, hq][rows]", "        s = s + 0 * bias[b, hq][rows]", 0),
    ("bias rows reversed", "        s = s + bias[b, hq][rows]",
     "        s = s + bias[b, hq][::-1][rows]", 0),
    ("identity normaliser one", "return np.full(n, NEG_INF), np.zeros(n), np.zeros((n, dv))",
     "return np.full(n, NEG_INF), np.ones(n), np.zeros((n, dv))", 0),
    ("monoid pairwise drops odd block", "                    if len(states) % 2:\n"
     "                        nxt.append(states[-1])",
     "                    if len(states) % 2 and False:\n"
     "                        nxt.append(states[-1])", 0),
    ("monoid left fold skips first block", "                for st in states:\n"
     "                    acc = merge(acc, st)",
     "                for st in states[1:]:\n"
     "                    acc = merge(acc, st)", 0),
    ("decode combine drops last split", "    for sp in range(n_splits):\n        st = merge(st,",
     "    for sp in range(n_splits - 1):\n        st = merge(st,", 0),
    ("decode ref keys and values swapped",
     "return decode_combine(*decode_partials(q, k, v, scale, n_splits))",
     "return decode_combine(*decode_partials(q, v, k, scale, n_splits))", 0),
    ("bias by key head", "        s = s + bias[b, hq][rows]", "        s = s + bias[b, hq // g][rows]",
     0),
]


def _load(src, name):
    mod = types.ModuleType(name)
    mod.__file__ = SRC_PATH
    exec(compile(src, SRC_PATH, "exec"), mod.__dict__)
    return mod


def _source():
    with open(SRC_PATH) as f:
        return f.read()


def test_unmutated_copy_passes_all_pins():
    mod = _load(_source(), "oracle_copy")
    for pin in P.ALL_PINS:
        pin(mod)


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ):
    src = _source()
    parts = src.split(old)
    assert len(parts) > occ + 1, f"mutation site not found: {old!r}"
    mutated = old.join(parts[:occ + 1]) + new + old.join(parts[occ + 1:])
    assert mutated != src
    mod = _load(mutated, "oracle_mutant")
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # a failing assertion or a crash both count
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"no pin caught mutant: {name}"
