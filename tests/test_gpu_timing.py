"""Per-kernel timing events (attn_set_timing_events): the events bound to
each kernel of a call record its start and end, in launch order, and a call
with events set computes exactly what a call without them does."""
import pytest
import torch

import attention_online_softmax_amd as aos
from attention_online_softmax_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:   # torch only reads elapsed times of events it has seen recorded
        e.record()
    torch.cuda.synchronize()
    return evs


def _check_spans(evs, n_kernels):
    spans = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(n_kernels)]
    assert all(s > 0 for s in spans), spans
    # kernel i + 1 starts after kernel i has ended (one stream)
    for i in range(n_kernels - 1):
        assert evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) >= 0


def test_timing_events_bwd_and_fwd():
    x = {k: v.cuda() for k, v in make_qkv(2, 4, 2, 300, 300, 128, seed=31, with_do=True).items()}
    o, lse = aos.attn_fwd(x["q"], x["k"], x["v"], causal=True)
    ref = aos.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True)
    evs = _events(4)
    aos.attn_set_timing_events([e.cuda_event for e in evs])
    try:
        o2, lse2 = aos.attn_fwd(x["q"], x["k"], x["v"], causal=True)
        torch.cuda.synchronize()
        _check_spans(evs, 1)
        got = aos.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True)
        torch.cuda.synchronize()
        _check_spans(evs, 2)
    finally:
        aos.attn_set_timing_events(None)
    assert torch.equal(o2, o) and torch.equal(lse2, lse)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_timing_events_decode():
    B, Hq, Hkv, Skv, d = 2, 8, 2, 1000, 128
    x = make_qkv(B, Hq, Hkv, 1, Skv, d, seed=32)
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    ref = aos.attn_decode(q, k, v, n_splits=4)
    evs = _events(4)
    aos.attn_set_timing_events([e.cuda_event for e in evs])
    try:
        got = aos.attn_decode(q, k, v, n_splits=4)
        torch.cuda.synchronize()
        _check_spans(evs, 2)
    finally:
        aos.attn_set_timing_events(None)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
