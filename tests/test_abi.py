"""C ABI contract checks that need no GPU.

The library must load, export every function include/attn.h declares, and
reject invalid arguments on the host before any HIP call (so these calls use
fake, never-dereferenced device addresses).
"""
import ctypes
import os
import re

import pytest

import attention_online_softmax_amd as aos

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(aos.LIB_PATH),
                                reason="libattn.so not built (run __graft_entry__.build())")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, HIP, VALUE = range(9)
F32, BF16 = 0, 1
MB = 1 << 20


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = aos.lib()
    names = declared_functions()
    assert set(names) == set(aos.EXPORTS), names
    for nm in names:
        assert hasattr(L, nm), f"missing export {nm}"


def test_version_and_strings():
    assert aos.attn_abi_version() == 5
    for s in range(9):
        assert aos.attn_status_str(s) and aos.attn_status_str(s) != "unknown status"
    assert aos.attn_status_str(99) == "unknown status"


def test_supports():
    for d in (64, 128, 256):
        assert aos.attn_supports(F32, 0, d) and aos.attn_supports(BF16, 0, d)
        assert aos.attn_supports(F32, 1, d) and aos.attn_supports(BF16, 1, d)
    assert aos.attn_supports(BF16, 2, 64) and aos.attn_supports(BF16, 2, 128)
    assert aos.attn_supports(BF16, 2, 256)           # the two-kernel backward at d256
    assert aos.attn_supports(BF16, 3, 64) and aos.attn_supports(BF16, 3, 128)
    assert not aos.attn_supports(BF16, 3, 256) and not aos.attn_supports(F32, 3, 128)
    assert aos.attn_supports(BF16, 4, 64) and aos.attn_supports(BF16, 4, 128)
    assert not aos.attn_supports(BF16, 4, 256) and not aos.attn_supports(F32, 4, 64)
    assert not aos.attn_supports(BF16, 0, 96)
    assert not aos.attn_supports(7, 0, 64)


def test_workspace_sizes():
    assert aos.attn_decode_workspace_bytes(8, 32, 128, 16) == 16 * 8 * 32 * 130 * 4
    assert aos.attn_decode_workspace_bytes(1, 1, 64, 1) == 512      # 66*4 rounded to 256
    assert aos.attn_decode_workspace_bytes(0, 1, 64, 1) == 0
    assert aos.attn_bwd_workspace_bytes(4, 16, 2048, 128) == 2 * 4 * 16 * 2048 * 4
    assert aos.attn_bwd_workspace_bytes(1, 1, 1, 64) == 256
    assert aos.attn_bwd_workspace_bytes(1, -1, 1, 64) == 0
    # fused: the pairs rounded up to 256 bytes, then the fp32 dQ accumulator
    assert aos.attn_bwd_fused_workspace_bytes(4, 16, 2048, 128) == \
        2 * 4 * 16 * 2048 * 4 + 4 * 16 * 2048 * 128 * 4
    assert aos.attn_bwd_fused_workspace_bytes(1, 1, 1, 64) == 256 + 256
    assert aos.attn_bwd_fused_workspace_bytes(1, 1, 3, 64) == 256 + 768
    assert aos.attn_bwd_fused_workspace_bytes(0, 1, 1, 64) == 0


class Fake:
    """Disjoint, 16-byte aligned fake device addresses (never dereferenced)."""

    def __init__(self):
        self.next = 1 << 40

    def __call__(self, nbytes=64 * MB):
        p = self.next
        self.next += nbytes + 4096
        return p


def fwd(dt=BF16, q=1, k=1, v=1, o=1, lse=1, B=1, Hq=2, Hkv=1, Sq=8, Skv=8, d=64, causal=0,
        scale=0.125, window=0, bias=None, sb=0, sh=0):
    return aos.lib().attn_fwd(dt, q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, d, causal, window, bias,
                              sb, sh, scale, None)


def test_fwd_validation():
    f = Fake()
    p = {n: f() for n in ("q", "k", "v", "o", "lse")}
    assert fwd(q=None, k=p["k"], v=p["v"], o=p["o"], lse=p["lse"]) == NULL
    base = dict(q=p["q"], k=p["k"], v=p["v"], o=p["o"], lse=p["lse"])
    assert fwd(**base, B=0) == SHAPE
    assert fwd(**base, Sq=0) == SHAPE
    assert fwd(**base, Hq=3, Hkv=2) == SHAPE
    assert fwd(**base, Sq=9, Skv=8, causal=1) == SHAPE
    assert fwd(**base, causal=0, window=4) == VALUE   # a window needs the causal mask
    bias = f()
    assert fwd(**base, bias=bias, Skv=6, Sq=6) == ALIGN     # rows of 6 floats: not 16-byte aligned
    assert fwd(**base, bias=bias + 4) == ALIGN
    assert fwd(**base, bias=bias, sb=6) == ALIGN
    assert fwd(**base, bias=bias, sh=-4) == VALUE
    assert fwd(**base, bias=p["o"]) == ALIAS                 # the bias overlaps an output
    assert fwd(**base, d=96) == UNSUP
    assert fwd(**base, dt=5) == UNSUP
    assert fwd(**base, scale=float("nan")) == VALUE
    assert fwd(**base, scale=float("inf")) == VALUE
    assert fwd(**dict(base, o=p["o"] + 8)) == ALIGN
    assert fwd(**dict(base, lse=p["lse"] + 4)) == ALIGN
    assert fwd(**dict(base, o=p["q"])) == ALIAS                        # output over input
    assert fwd(**dict(base, o=p["q"] + 16 * 64 * 2 - 16)) == ALIAS     # partial overlap
    assert fwd(**dict(base, lse=p["o"] + 16)) == ALIAS                 # outputs overlap
    assert fwd(**base, Sq=1 << 30, Skv=1 << 30) == SHAPE               # beyond 32-bit per head


def test_decode_validation():
    f = Fake()
    q, k, v, o, lse, ws = (f() for _ in range(6))
    need = aos.attn_decode_workspace_bytes(2, 8, 128, 16)
    L = aos.lib()

    def call(**kw):
        a = dict(dt=BF16, q=q, k=k, v=v, o=o, lse=lse, B=2, Hq=8, Hkv=2, Skv=4096, d=128,
                 scale=0.1, n=16, ws=ws, wsb=need)
        a.update(kw)
        return L.attn_decode(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                             a["Hkv"], a["Skv"], a["d"], a["scale"], a["n"], a["ws"], a["wsb"],
                             None)

    assert call(k=None) == NULL
    assert call(Hq=6, Hkv=4) == SHAPE
    assert call(Skv=0) == SHAPE
    assert call(d=80) == UNSUP
    assert call(n=0) == VALUE
    assert call(n=257) == VALUE
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=ws + 8) == ALIGN
    assert call(ws=k) == ALIAS
    assert call(o=q) == ALIAS
    assert call(scale=float("-inf")) == VALUE


def test_decode_noalloc_validation():
    """attn_decode_noalloc rejects bad arguments, and problems whose split
    states exceed the static scratch, before touching the device."""
    f = Fake()
    q, k, v, o, lse = (f() for _ in range(5))
    L = aos.lib()

    def call(**kw):
        a = dict(dt=BF16, q=q, k=k, v=v, o=o, lse=lse, B=2, Hq=8, Hkv=2, Skv=4096, d=128,
                 scale=0.1, n=16)
        a.update(kw)
        return L.attn_decode_noalloc(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                     a["Hq"], a["Hkv"], a["Skv"], a["d"], a["scale"], a["n"], None)

    assert call(k=None) == NULL
    assert call(Hq=6, Hkv=4) == SHAPE
    assert call(d=80) == UNSUP
    assert call(n=0) == VALUE
    assert call(scale=float("nan")) == VALUE
    assert call(o=q) == ALIAS
    assert call(q=q + 8) == ALIGN
    # 256 splits x 64 x 64 heads x 130 floats: 545 MB of split states
    assert aos.attn_decode_workspace_bytes(64, 64, 128, 256) > aos.binding.SCRATCH_BYTES
    assert call(B=64, Hq=64, Hkv=8, n=256) == WS
    assert "static scratch" in aos.attn_status_str(WS)


def test_fwd_tile_entry_points():
    """Tile override: all of (nw, bc, split) zero, or all positive with
    split dividing nw; plan: unsupported head dims and invalid shapes list
    nothing (both checks happen before any device query)."""
    L = aos.lib()
    assert L.attn_fwd_tile_override(4, 0, 1) == VALUE
    assert L.attn_fwd_tile_override(0, 32, 1) == VALUE
    assert L.attn_fwd_tile_override(4, 32, 0) == VALUE
    assert L.attn_fwd_tile_override(-4, 32, 1) == VALUE
    assert L.attn_fwd_tile_override(4, -32, 1) == VALUE
    assert L.attn_fwd_tile_override(4, 32, 3) == VALUE      # 3 key groups of 4 waves
    assert L.attn_fwd_tile_override(4, 32, 4) == 0
    assert L.attn_fwd_tile_override(4, 64, 2) == 0
    assert L.attn_fwd_tile_override(0, 0, 0) == 0
    assert aos.attn_fwd_tile_plan(80, True, 1, 1, 1, 64, 64) == (None, [])
    assert aos.attn_fwd_tile_plan(128, True, 1, 3, 2, 64, 64) == (None, [])
    assert aos.attn_fwd_tile_plan(128, True, 1, 2, 2, 65, 64) == (None, [])


def test_bwd_tile_override_values():
    """Backward launch shapes: (0, 0), (4, 1), (4, 2) and (2, 4) only, for
    dK/dV and for dQ; the head split 0 to 8."""
    L = aos.lib()
    good = ((4, 1), (4, 2), (2, 4), (0, 0))
    for a in good:
        for b in good:
            assert L.attn_bwd_tile_override(*a, *b, 0) == 0
    for p in range(9):
        assert L.attn_bwd_tile_override(0, 0, 0, 0, p) == 0
    for p in (-1, 9, 16):
        assert L.attn_bwd_tile_override(0, 0, 0, 0, p) == VALUE
    for bad in ((2, 2), (4, 4), (8, 1), (0, 1), (4, 0), (-4, 1), (1, 8)):
        assert L.attn_bwd_tile_override(*bad, 0, 0, 0) == VALUE
        assert L.attn_bwd_tile_override(0, 0, *bad, 0) == VALUE
    assert L.attn_bwd_tile_override(0, 0, 0, 0, 0) == 0


def test_bwd_split_workspace_bytes():
    """The split workspace is at least the plain one, a multiple of 256 bytes,
    the plain one for shapes that never split (no grouped heads
    to deal out, or grids that fill the device), and 0 for invalid sizes."""
    plain = aos.attn_bwd_workspace_bytes(1, 32, 4096, 128)
    split = aos.attn_bwd_split_workspace_bytes(1, 32, 4, 4096, 4096, 128, True)
    assert split >= plain and split % 256 == 0
    # eight query heads per key/value head over 32 key tiles: the split pays
    nkv = 1 * 4 * 4096 * 128
    assert split > plain and (split - plain) % (2 * nkv * 4) < 256
    # one query head per key/value head: nothing to split
    assert (aos.attn_bwd_split_workspace_bytes(1, 8, 8, 2048, 2048, 128, True) ==
            aos.attn_bwd_workspace_bytes(1, 8, 2048, 128))
    assert aos.attn_bwd_split_workspace_bytes(0, 8, 8, 64, 64, 128, True) == 0
    assert aos.attn_bwd_split_workspace_bytes(1, 8, 3, 64, 64, 128, True) == 0
    assert aos.attn_bwd_split_workspace_bytes(1, 8, 8, 65, 64, 128, True) == 0


def test_decode_paged_validation():
    f = Fake()
    q, kp, vp, tab, lens, o, lse, ws = (f() for _ in range(8))
    need = aos.attn_decode_workspace_bytes(2, 8, 128, 16)
    L = aos.lib()

    def call(**kw):
        a = dict(dt=BF16, q=q, kp=kp, vp=vp, tab=tab, lens=lens, o=o, lse=lse, B=2, Hq=8, Hkv=2,
                 d=128, npg=64, ps=64, mp=32, scale=0.1, n=16, ws=ws, wsb=need)
        a.update(kw)
        return L.attn_decode_paged(a["dt"], a["q"], a["kp"], a["vp"], a["tab"], a["lens"],
                                   a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["d"], a["npg"],
                                   a["ps"], a["mp"], a["scale"], a["n"], a["ws"], a["wsb"], None)

    assert call(tab=None) == NULL
    assert call(lens=None) == NULL
    assert call(kp=None) == NULL
    assert call(npg=0) == SHAPE
    assert call(mp=0) == SHAPE
    assert call(ps=0) == SHAPE
    assert call(Hq=6, Hkv=4) == SHAPE
    assert call(dt=F32) == UNSUP
    assert call(d=256) == UNSUP
    assert call(ps=48) == VALUE                      # pages hold whole 32-key tiles
    assert call(mp=1 << 26, ps=64) == SHAPE          # 2^32 keys per stream
    assert call(n=0) == VALUE
    assert call(n=257) == VALUE
    assert call(scale=float("nan")) == VALUE
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(tab=tab + 2) == ALIGN
    assert call(lens=lens + 1) == ALIGN
    assert call(q=q + 8) == ALIGN
    assert call(o=kp) == ALIAS
    assert call(ws=tab) == ALIAS
    assert call(lse=vp + 64) == ALIAS


def test_bwd_validation():
    f = Fake()
    names = ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws")
    p = {n: f() for n in names}
    need = aos.attn_bwd_workspace_bytes(1, 4, 64, 128)
    L = aos.lib()

    def call(**kw):
        a = dict(p)
        a.update(dict(dt=BF16, B=1, Hq=4, Hkv=2, Sq=64, Skv=64, d=128, causal=1, window=0,
                      bias=None, sb=0, sh=0, scale=0.1, wsb=need))
        a.update(kw)
        return L.attn_bwd(a["dt"], a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                          a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["d"],
                          a["causal"], a["window"], a["bias"], a["sb"], a["sh"], a["scale"],
                          a["ws"], a["wsb"], None)

    for n in names[:-1]:
        assert call(**{n: None}) == NULL, n
    assert call(Sq=65) == SHAPE
    assert call(Hq=5) == SHAPE
    assert call(d=96) == UNSUP
    assert call(dt=F32) == UNSUP
    assert call(ws=None) == WS
    assert call(wsb=16) == WS
    assert call(dk=p["dv"]) == ALIAS
    assert call(dq=p["do"]) == ALIAS
    assert call(ws=p["lse"]) == ALIAS
    assert call(dv=p["dv"] + 2) == ALIGN
    assert call(causal=0, window=16) == VALUE        # a window needs the causal mask
    assert call(bias=p["ws"]) == ALIAS               # the bias overlaps the workspace
    assert call(bias=f() + 8) == ALIGN
    assert call(bias=f(), sb=-8) == VALUE


def test_bwd_fused_validation():
    f = Fake()
    names = ("q", "k", "v", "o", "do", "lse", "dq", "dk", "dv", "ws")
    p = {n: f() for n in names}
    need = aos.attn_bwd_fused_workspace_bytes(1, 4, 64, 128)
    L = aos.lib()

    def call(**kw):
        a = dict(p)
        a.update(dict(dt=BF16, B=1, Hq=4, Hkv=2, Sq=64, Skv=64, d=128, causal=1, window=0,
                      bias=None, sb=0, sh=0, scale=0.1, wsb=need))
        a.update(kw)
        return L.attn_bwd_fused(a["dt"], a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"],
                                a["dq"], a["dk"], a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                                a["Skv"], a["d"], a["causal"], a["window"], a["bias"], a["sb"],
                                a["sh"], a["scale"], a["ws"], a["wsb"], None)

    for n in names[:-1]:
        assert call(**{n: None}) == NULL, n
    assert call(Sq=65) == SHAPE
    assert call(Hq=5) == SHAPE
    assert call(B=0) == SHAPE
    assert call(d=256) == UNSUP
    assert call(dt=F32) == UNSUP
    assert call(scale=float("nan")) == VALUE
    assert call(ws=None) == WS
    assert call(wsb=need - 256) == WS        # room for the pairs but not the accumulator
    assert call(dk=p["dv"]) == ALIAS
    assert call(dq=p["do"]) == ALIAS
    assert call(ws=p["lse"]) == ALIAS
    assert call(dv=p["dv"] + 2) == ALIGN
    assert call(ws=p["ws"] + 8) == ALIGN
    assert call(causal=0, window=16) == VALUE   # a window needs the causal mask
    assert call(bias=f(), sb=-8) == VALUE
    assert call(bias=p["dq"]) == ALIAS           # dQ written over the bias read


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import attention_online_softmax_amd.binding as bnd
    monkeypatch.setattr(bnd, "_lib", None)
    monkeypatch.setattr(bnd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bnd.lib()


# The backward's launch choices measured fastest on MI355X (256 compute
# units, which the plan assumes without a device): (B, Hq, Hkv, S, d, causal)
# -> dK/dV shape, dQ shape, with the plain workspace (no head split).
BWD_SHAPE_PICKS = [
    ((1, 32, 4, 4096, 128, True), (2, 4), (4, 1)),
    ((1, 16, 2, 2048, 128, True), (2, 4), (2, 4)),
    ((1, 8, 1, 8192, 128, True), (2, 4), (4, 1)),
    ((1, 64, 8, 6144, 128, True), (2, 4), (4, 1)),
    ((2, 16, 4, 4096, 128, True), (2, 4), (4, 1)),
    ((2, 32, 8, 1024, 64, True), (2, 4), (4, 1)),
    ((4, 32, 8, 4096, 128, True), (4, 1), (4, 1)),
    ((2, 8, 8, 1024, 64, True), (2, 4), (2, 4)),
    ((2, 16, 16, 512, 128, True), (2, 4), (2, 4)),
    ((1, 12, 12, 2048, 128, True), (2, 4), (2, 4)),
    ((2, 16, 16, 1536, 128, True), (4, 2), (4, 1)),
    ((2, 16, 16, 2048, 128, True), (4, 2), (4, 1)),
    ((1, 16, 16, 2048, 128, False), (4, 2), (4, 1)),
    ((3, 16, 16, 2048, 128, True), (4, 1), (4, 1)),
    ((1, 40, 40, 2048, 128, True), (4, 1), (4, 1)),
    ((4, 16, 16, 2048, 128, True), (4, 1), (4, 1)),
    ((8, 16, 16, 2048, 64, True), (4, 1), (4, 1)),
    ((1, 32, 32, 2048, 64, False), (4, 1), (4, 1)),
]

# The head split with the workspace of attn_bwd_split_workspace_bytes: the
# split the library takes, each within run-to-run noise of the fastest
# measured on MI355X.
BWD_SPLIT_PICKS = [
    ((1, 16, 2, 2048, 128, True), 8),
    ((1, 32, 4, 4096, 128, True), 4),
    ((2, 32, 4, 4096, 128, True), 4),
    ((4, 32, 4, 4096, 128, True), 4),
    ((1, 16, 2, 4096, 128, False), 8),
    ((1, 32, 8, 2048, 64, True), 2),
    ((2, 16, 2, 4096, 256, True), 4),
    ((1, 16, 2, 8192, 256, True), 4),
    ((1, 64, 8, 4096, 128, True), 4),
    ((4, 16, 16, 2048, 128, True), 1),
]


@pytest.mark.parametrize("shape,kv,q", BWD_SHAPE_PICKS, ids=lambda v: str(v))
def test_bwd_plan_wave_groups(shape, kv, q):
    B, Hq, Hkv, S, d, causal = shape
    plain = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    plan = aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, causal, workspace_bytes=plain)
    assert plan == {"dkdv": kv, "dq": q, "hsplit": 1}


@pytest.mark.parametrize("shape,p", BWD_SPLIT_PICKS, ids=lambda v: str(v))
def test_bwd_plan_head_split(shape, p):
    B, Hq, Hkv, S, d, causal = shape
    plan = aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, causal)
    assert plan["hsplit"] == p
    if d > 128:
        assert plan["dkdv"] == (4, 1) and plan["dq"] == (4, 1)
    # the split workspace holds exactly the pairs and p float32 copies of dK, dV
    plain = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    split = aos.attn_bwd_split_workspace_bytes(B, Hq, Hkv, S, S, d, causal)
    want = plain if p == 1 else (plain + 255) // 256 * 256 + p * 2 * B * Hkv * S * d * 4
    assert split == (want + 255) // 256 * 256 if p > 1 else split == plain


def test_bwd_plan_never_splits():
    """No split with a window, a bias, the plain workspace or one query head
    per key/value head."""
    B, Hq, Hkv, S, d = 1, 16, 2, 2048, 128
    big = 1 << 34
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=big)["hsplit"] > 1
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, window=512, workspace_bytes=big)["hsplit"] == 1
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, bias=True, workspace_bytes=big)["hsplit"] == 1
    plain = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=plain)["hsplit"] == 1
    assert aos.attn_bwd_plan(1, 8, 8, S, S, d, True, workspace_bytes=big)["hsplit"] == 1
    # a window of at least Skv keys is no window
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, window=S,
                             workspace_bytes=big)["hsplit"] > 1


def test_bwd_plan_override_and_errors():
    B, Hq, Hkv, S, d = 1, 16, 2, 1024, 128
    big = 1 << 34
    plain = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
    aos.attn_bwd_tile_override(4, 2, 2, 4, 3)
    try:
        assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=big) == {
            "dkdv": (4, 2), "dq": (2, 4), "hsplit": 3}
        # a forced split the workspace cannot hold
        with pytest.raises(aos.AttnError) as e:
            aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=plain)
        assert e.value.status == 6
        # d = 256 keeps the plain shapes, forced or not
        assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, 256, True, workspace_bytes=big) == {
            "dkdv": (4, 1), "dq": (4, 1), "hsplit": 3}
    finally:
        aos.attn_bwd_tile_override(0, 0, 0, 0, 0)
    assert aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=big)["hsplit"] == 8
    for kw, status in ((dict(Hkv=3), 2), (dict(d=96), 3), (dict(causal=False, window=64), 8),
                       (dict(ws=plain - 16), 6), (dict(Sq=S + 1), 2)):
        a = dict(B=B, Hq=Hq, Hkv=Hkv, Sq=S, Skv=S, d=d, causal=True, window=0, ws=big)
        a.update(kw)
        with pytest.raises(aos.AttnError) as e:
            aos.attn_bwd_plan(a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["d"], a["causal"],
                              window=a["window"], workspace_bytes=a["ws"])
        assert e.value.status == status, kw
    L = aos.lib()
    import ctypes
    x = ctypes.c_int()
    assert L.attn_bwd_plan(B, Hq, Hkv, S, S, d, 1, 0, 0, big, None, ctypes.byref(x),
                           ctypes.byref(x), ctypes.byref(x), ctypes.byref(x)) == 1
