"""attn_decode_noalloc (split states in the library's static device scratch)
against attn_decode (caller workspace) and the float64 oracle, on calls in a
row whose second input is smaller than the first, so that the scratch still
holds the first call's states when the second runs."""
import math

import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, inputs, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, Skv, d, n_splits, dtype): the grouped-query decode shape
# first, then smaller ones on the matrix-core and the vector-unit kernels.
SEQUENCES = [
    [(8, 32, 8, 4096, 128, 16, "bf16"), (2, 8, 2, 1000, 128, 5, "bf16")],
    [(2, 8, 2, 3000, 64, 16, "f32"), (1, 4, 1, 77, 64, 3, "f32")],
    [(2, 16, 4, 2048, 256, 8, "bf16"), (1, 2, 2, 300, 64, 16, "bf16")],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: f"{s[0][6]}_d{s[0][4]}")
def test_noalloc_matches_workspace_entry_point(seq):
    for i, case in enumerate(seq):
        B, Hq, Hkv, Skv, d, n, dt = case
        dev, ref = inputs(B, Hq, Hkv, 1, Skv, d, dt, 9000 + 17 * i + sum(case[:6]))
        scale = 1 / math.sqrt(d)
        o_na = torch.full_like(dev["q"], float("nan"))
        l_na = torch.full((B, Hq, 1), float("nan"), device="cuda")
        note(f"noalloc call {i}: {case}")
        aos.attn_decode_noalloc(dev["q"], dev["k"], dev["v"], scale=scale, n_splits=n, o=o_na,
                                lse=l_na)
        o_ws, l_ws = aos.attn_decode(dev["q"], dev["k"], dev["v"], scale=scale, n_splits=n)
        torch.cuda.synchronize()
        # The same kernels on the same inputs: identical bits.
        assert torch.equal(o_na, o_ws), f"call {i}: O differs from attn_decode"
        assert torch.equal(l_na, l_ws), f"call {i}: LSE differs from attn_decode"
        O, L = oracle.decode_ref(ref["q"], ref["k"], ref["v"], scale, n)
        assert_close(to_f64(o_na), O, TOL_O[dt], f"call {i} O")
        assert_close(l_na.cpu().numpy(), L, TOL_LSE[dt], f"call {i} LSE")


def test_noalloc_rejects_too_large():
    """A problem whose split states exceed the static scratch raises before
    anything is launched (outputs untouched)."""
    B, Hq, Hkv, Skv, d, n = 64, 64, 8, 64, 128, 256
    assert aos.attn_decode_workspace_bytes(B, Hq, d, n) > aos.binding.SCRATCH_BYTES
    dev, _ = inputs(B, Hq, Hkv, 1, Skv, d, "bf16", 9100)
    o = torch.full_like(dev["q"], 7.0)
    with pytest.raises(aos.AttnError):
        aos.attn_decode_noalloc(dev["q"], dev["k"], dev["v"], n_splits=n, o=o)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
