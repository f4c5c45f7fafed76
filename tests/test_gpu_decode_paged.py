"""Paged, variable-length decode through the C ABI against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
import oracle
from attention_online_softmax_amd.inputs import PAGED_WORKLOAD, make_paged, make_qkv, to_f64
from tests.gpu_util import TOL_LSE, TOL_O, assert_close, note

pytestmark = pytest.mark.gpu

# (B, Hq, Hkv, d, page_size, max_pages, lens, n_splits): grouped heads from 1
# to 16 per key/value head, pages of 32 to 256 keys, ragged lengths (0, 1,
# around a tile and a page boundary), more splits than tiles, lengths past
# the table's capacity (clamped) and negative (empty).
CASES = [
    (3, 8, 2, 128, 64, 8, [512, 100, 1], 16),
    (4, 4, 4, 64, 32, 10, [0, 31, 32, 33], 3),
    (2, 16, 1, 128, 256, 4, [1000, 700], 7),
    (2, 8, 8, 64, 128, 3, [384, 200], 1),
    (1, 32, 8, 128, 32, 40, [1280], 64),
    (2, 4, 1, 128, 64, 5, [10 ** 6, -3], 4),
]


def run_case(dev, scale, n_splits):
    o, lse = aos.attn_decode_paged(dev["q"], dev["k_pages"], dev["v_pages"], dev["block_table"],
                                   dev["seq_lens"], scale=scale, n_splits=n_splits)
    torch.cuda.synchronize()
    return o, lse


def check(o, lse, cpu, scale, what):
    ref = {k: (to_f64(v) if v.is_floating_point() else v.numpy()) for k, v in cpu.items()}
    O, L = oracle.decode_paged_ref(ref["q"], ref["k_pages"], ref["v_pages"], ref["block_table"],
                                   ref["seq_lens"], scale)
    got_o, got_l = to_f64(o), lse.cpu().numpy().astype(np.float64)
    empty = np.isinf(L)
    assert np.array_equal(np.isinf(got_l), empty), f"{what}: empty streams differ"
    assert np.all(got_l[empty] < 0), f"{what}: empty-stream LSE must be -inf"
    assert np.all(got_o[np.broadcast_to(empty[..., None], got_o.shape)] == 0), f"{what}: empty O"
    assert_close(got_o, O, TOL_O["bf16"], f"{what} O")
    assert_close(np.where(empty, 0, got_l), np.where(empty, 0, L), TOL_LSE["bf16"], f"{what} LSE")


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B{}_Hq{}_Hkv{}_d{}_ps{}_mp{}_n{}".format(
    *c[:6], c[7]))
def test_paged_parity(case):
    B, Hq, Hkv, d, ps, mp, lens, n = case
    cpu = make_paged(B, Hq, Hkv, d, ps, mp, lens, seed=700 + B * 10 + d)
    dev = {k: v.cuda() for k, v in cpu.items()}
    scale = 1 / math.sqrt(d)
    note(f"paged decode {case}")
    o, lse = run_case(dev, scale, n)
    check(o, lse, cpu, scale, f"paged {case}")


def test_paged_shared_and_invalid_pages():
    """Streams sharing prefix pages, and page ids outside the pool (which
    read as zeros)."""
    B, Hq, Hkv, d, ps, mp = 3, 8, 2, 128, 64, 6
    cpu = make_paged(B, Hq, Hkv, d, ps, mp, [384, 300, 250], seed=777)
    t = cpu["block_table"]
    t[1, :2] = t[0, :2]            # streams 0 and 1 share their first two pages
    t[2, 1] = -1                   # outside the pool
    t[2, 3] = cpu["k_pages"].shape[0] + 5
    dev = {k: v.cuda() for k, v in cpu.items()}
    note("paged decode shared / invalid pages")
    o, lse = run_case(dev, 1 / math.sqrt(d), 16)
    check(o, lse, cpu, 1 / math.sqrt(d), "paged shared/invalid")


@pytest.mark.parametrize("d", [64, 128])
def test_paged_identity_equals_contiguous(d):
    """Pages laid out in order with full lengths: the same tiles in the same
    order as attn_decode on the contiguous cache, so the outputs are equal
    bit for bit."""
    B, Hq, Hkv, S, ps = 2, 8, 2, 1000, 64
    mp = (S + ps - 1) // ps
    cpu = make_qkv(B, Hq, Hkv, 1, mp * ps, d, torch.bfloat16, 880 + d)
    k, v = cpu["k"], cpu["v"]

    def pool(x):  # page b * mp + i holds keys [i ps, (i + 1) ps) of stream b
        return x.reshape(B, Hkv, mp, ps, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, d)

    dev = {"q": cpu["q"].cuda(), "k_pages": pool(k).contiguous().cuda(),
           "v_pages": pool(v).contiguous().cuda(),
           "block_table": torch.arange(B * mp, dtype=torch.int32).reshape(B, mp).cuda(),
           "seq_lens": torch.full((B,), S, dtype=torch.int32).cuda()}
    note(f"paged identity vs contiguous d={d}")
    o, lse = run_case(dev, 1 / math.sqrt(d), 16)
    oc, lc = aos.attn_decode(cpu["q"].cuda(), k[:, :, :S].contiguous().cuda(),
                             v[:, :, :S].contiguous().cuda(), n_splits=16)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)


def test_paged_workload_full():
    w = PAGED_WORKLOAD
    cpu = make_paged(w["B"], w["Hq"], w["Hkv"], w["d"], w["page_size"], w["max_pages"], w["lens"],
                     seed=w["seed"])
    dev = {k: v.cuda() for k, v in cpu.items()}
    scale = 1 / math.sqrt(w["d"])
    note("paged decode workload")
    o, lse = run_case(dev, scale, w["n_splits"])
    check(o, lse, cpu, scale, "paged workload")
