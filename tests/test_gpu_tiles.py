"""Every compiled tile candidate of the bf16 forward (waves per workgroup,
keys per tile), forced through attn_fwd_tile_override, against the float64
oracle; and the estimate's plan ("Tang, a compiler that derives GPU kernels
and bounds how fast they can run", Abstract: a per-tile estimate picks the
tile)."""
import math

import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu

CANDS = {64: [(4, 64, 1), (4, 32, 1), (8, 64, 1), (2, 64, 1), (4, 32, 4), (2, 32, 2), (4, 64, 2)],
         128: [(4, 32, 1), (4, 64, 1), (8, 32, 1), (8, 64, 1), (4, 32, 4), (2, 32, 2), (4, 32, 2)],
         256: [(8, 32, 1), (4, 32, 1)]}
# (B, Hq, Hkv, Sq, Skv, causal): ragged tails, grouped heads, Sq < Skv.
SHAPES = [(1, 4, 2, 300, 300, True), (2, 2, 1, 77, 333, False), (1, 2, 2, 200, 460, True)]


@pytest.mark.parametrize("d", [64, 128, 256])
def test_plan_lists_the_compiled_candidates(d):
    pick, cands = aos.attn_fwd_tile_plan(d, True, 4, 16, 16, 2048, 2048)
    assert [(c["nw"], c["bc"], c["split"]) for c in cands] == CANDS[d]
    assert 0 <= pick < len(cands)
    # The key-split candidates (one 32-row block, split = nw) apply only to
    # grids of at most one such block per compute unit; every other
    # candidate has an estimate.
    for c in cands:
        if c["split"] < c["nw"]:
            assert c["est_us"] > 0 and math.isfinite(c["est_us"])
        else:
            assert c["est_us"] is None
    est = [c["est_us"] if c["est_us"] is not None else math.inf for c in cands]
    assert pick == min(range(len(cands)), key=lambda i: est[i])


@pytest.mark.parametrize("d", [64, 128])
def test_plan_key_split_on_a_tiny_grid(d):
    # 8 query blocks x 8 heads: 64 workgroups of the key-split kernel, far
    # fewer than compute units; it gets an estimate there.
    pick, cands = aos.attn_fwd_tile_plan(d, False, 1, 8, 8, 256, 256)
    ks = [c for c in cands if c["split"] == c["nw"]]
    assert ks and all(c["est_us"] is not None and c["est_us"] > 0 for c in ks)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}_Hq{}_Hkv{}_Sq{}_Skv{}_{}".format(
    *s[:5], "causal" if s[5] else "full"))
def test_every_candidate_parity(d, shape):
    B, Hq, Hkv, Sq, Skv, causal = shape
    dev, ref = inputs(B, Hq, Hkv, Sq, Skv, d, "bf16", 600 + d + Sq)
    scale = 1 / math.sqrt(d)
    O, L = oracle.attention_ref(ref["q"], ref["k"], ref["v"], causal, scale)
    for nw, bc, sp in CANDS[d]:
        note(f"tile candidate nw{nw} bc{bc} split{sp} d{d} {shape}")
        aos.attn_fwd_tile_override(nw, bc, sp)
        try:
            o, lse = aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=causal, scale=scale)
            torch.cuda.synchronize()
        finally:
            aos.attn_fwd_tile_override(0, 0)
        assert_close(to_f64(o), O, TOL_O["bf16"], f"nw{nw} bc{bc} split{sp} O")
        assert_close(lse.cpu().numpy(), L, TOL_LSE["bf16"], f"nw{nw} bc{bc} split{sp} LSE")


def test_override_not_compiled_is_rejected():
    dev, _ = inputs(1, 2, 2, 64, 64, 256, "bf16", 5)
    aos.attn_fwd_tile_override(2, 64, 1)   # not a d256 candidate
    try:
        with pytest.raises(aos.AttnError):
            aos.attn_fwd(dev["q"], dev["k"], dev["v"], causal=True)
    finally:
        aos.attn_fwd_tile_override(0, 0)
    with pytest.raises(aos.AttnError):
        aos.attn_fwd_tile_override(4, 0)
