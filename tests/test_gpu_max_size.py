"""Decode, and the forward with one query row, at the largest per-head size
the ABI accepts (Skv * d just below 2^31 elements, so K and V are 4-8 GiB
per tensor and byte offsets pass 2^32).  The float64 reference is the definition of the attention evaluated
on the inputs' structure: every key row is zero except a few "spike" rows,
so the scores are 0 except at the spikes and

    O = (sum_spikes e^(s_j - M) V_j + e^-M (sum_all V - sum_spikes V))
        / (sum_spikes e^(s_j - M) + (Skv - #spikes) e^-M),
    LSE = M + ln(denominator),  M = max(0, max_j s_j),

with the sum over all V rows taken in float64 on the host.  A spike read
from a wrong row, a lost split or a wrapped 32-bit offset moves O by about
the size of a V row."""
import math

import numpy as np
import pytest
import torch

import attention_online_softmax_amd as aos
from attention_online_softmax_amd.inputs import randn, to_f64
from tests.gpu_util import TOL_GRAD, TOL_LSE, TOL_O, assert_close, note

pytestmark = pytest.mark.gpu


def v_sum_f64(v):
    """Sum of the rows of v [1, 1, S, d] (GPU) in float64 on the host, in
    chunks of 2^20 rows."""
    S = v.shape[2]
    tot = np.zeros(v.shape[3], dtype=np.float64)
    for r0 in range(0, S, 1 << 20):
        tot += to_f64(v[0, 0, r0:r0 + (1 << 20)]).sum(axis=0)
    return tot


def run_case(dt, d, Skv, Hq, n_splits, seed, entry="decode"):
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    note(f"max-size decode {dt} d{d} Skv{Skv} Hq{Hq} splits{n_splits}: inputs")
    q = randn((1, Hq, 1, d), seed, 1.0, tdt).cuda()
    k = torch.zeros((1, 1, Skv, d), device="cuda", dtype=tdt)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    v = torch.randn((1, 1, Skv, d), device="cuda", dtype=torch.float32, generator=g).to(tdt) \
        if dt != "f32" else torch.randn((1, 1, Skv, d), device="cuda", dtype=tdt, generator=g)
    spikes = {0: 1.5, 12345: 1.7, (1 << 23) + 7: 1.9, Skv - 33: 2.0, Skv - 1: 2.1}
    for j, c in spikes.items():
        k[0, 0, j] = (q[0, 0, 0].float() * c).to(tdt)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(d)
    note(f"max-size {entry} {dt} d{d} Skv{Skv}: run")
    if entry == "decode":
        o, lse = aos.attn_decode(q, k, v, scale=scale, n_splits=n_splits)
    else:
        o, lse = aos.attn_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    note(f"max-size {entry} {dt} d{d} Skv{Skv}: float64 reference")
    qf = to_f64(q)[0, :, 0]                                   # [Hq, d]
    ks = {j: to_f64(k[0, 0, j]) for j in spikes}
    vs = {j: to_f64(v[0, 0, j]) for j in spikes}
    v_rest = v_sum_f64(v) - sum(vs.values())
    n_rest = Skv - len(spikes)
    O = np.zeros((Hq, d))
    L = np.zeros(Hq)
    for h in range(Hq):
        s = {j: scale * float(qf[h] @ ks[j]) for j in spikes}
        M = max(0.0, max(s.values()))
        num = sum(math.exp(s[j] - M) * vs[j] for j in spikes) + math.exp(-M) * v_rest
        den = sum(math.exp(s[j] - M) for j in spikes) + n_rest * math.exp(-M)
        O[h] = num / den
        L[h] = M + math.log(den)
    # head 0's spikes dominate its softmax: O there is close to a mix of
    # the spike rows, so a wrong spike row shows at full size
    assert_close(to_f64(o)[0, :, 0], O, TOL_O[dt], f"max-size {entry} {dt} O")
    assert_close(lse.cpu().numpy()[0, :, 0], L, TOL_LSE[dt], f"max-size {entry} {dt} LSE")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("n_splits", [16, 256])
def test_decode_max_size_bf16(n_splits):
    """bf16, d = 128 (matrix-core split kernel), Skv = 2^24 - 32: 4 GiB per
    cache tensor, Skv * d = 2^31 - 4096."""
    run_case("bf16", 128, (1 << 24) - 32, 8, n_splits, 4100 + n_splits)


def test_decode_max_size_f32():
    """float32, d = 64 (vector split kernel), Skv = 2^25 - 64: 8 GiB per cache
    tensor, Skv * d = 2^31 - 4096."""
    run_case("f32", 64, (1 << 25) - 64, 4, 16, 4300)


@pytest.mark.parametrize("dt,d,Skv", [("bf16", 128, (1 << 24) - 32), ("f32", 64, (1 << 25) - 64)])
def test_fwd_one_row_max_size(dt, d, Skv):
    """attn_fwd with a single query row (causal, bottom-right aligned: it sees
    every key) over the largest key count per head."""
    run_case(dt, d, Skv, 8 if dt == "bf16" else 4, 0, 4500 + d, entry="fwd")


@pytest.mark.parametrize("fused", [False, True], ids=["two_kernel", "fused"])
def test_bwd_one_row_max_size(fused):
    """Backward of one query row over 2^24 - 32 keys (bf16, d = 128, causal,
    bottom-right aligned).  With the spike structure the gradients have
    closed forms: P_j = e^(s_j - M) / den, dV_j = P_j dO, dS_j = P_j (dO.V_j -
    dO.O), dK_j = scale dS_j q, dQ = scale sum_spikes dS_j K_j (the other key
    rows are zero).  dV and dK are checked on the spike rows, the first and
    last rows and 64 seeded random rows; dQ in full."""
    d, Skv, seed = 128, (1 << 24) - 32, 4700
    tdt = torch.bfloat16
    note(f"max-size bwd fused={fused}: inputs")
    q = randn((1, 1, 1, d), seed, 1.0, tdt).cuda()
    do = randn((1, 1, 1, d), seed + 3, 1.0, tdt).cuda()
    k = torch.zeros((1, 1, Skv, d), device="cuda", dtype=tdt)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    v = torch.randn((1, 1, Skv, d), device="cuda", dtype=torch.float32, generator=g).to(tdt)
    spikes = {0: 1.5, 12345: 1.7, (1 << 23) + 7: 1.9, Skv - 33: 2.0, Skv - 1: 2.1}
    for j, c in spikes.items():
        k[0, 0, j] = (q[0, 0, 0].float() * c).to(tdt)
    scale = 1 / math.sqrt(d)
    note(f"max-size bwd fused={fused}: forward + backward")
    o, lse = aos.attn_fwd(q, k, v, causal=True, scale=scale)
    bwd = aos.attn_bwd_fused if fused else aos.attn_bwd
    dq, dk, dv = bwd(q, k, v, o, do, lse, causal=True, scale=scale)
    torch.cuda.synchronize()
    note(f"max-size bwd fused={fused}: float64 reference")
    qf, dof = to_f64(q)[0, 0, 0], to_f64(do)[0, 0, 0]
    ks = {j: to_f64(k[0, 0, j]) for j in spikes}
    vs = {j: to_f64(v[0, 0, j]) for j in spikes}
    v_all = v_sum_f64(v)
    n_rest = Skv - len(spikes)
    s = {j: scale * float(qf @ ks[j]) for j in spikes}
    M = max(0.0, max(s.values()))
    den = sum(math.exp(s[j] - M) for j in spikes) + n_rest * math.exp(-M)
    p = {j: math.exp(s[j] - M) / den for j in spikes}
    p_rest = math.exp(-M) / den
    O = sum(p[j] * vs[j] for j in spikes) + p_rest * (v_all - sum(vs.values()))
    Dd = float(dof @ O)
    rng = np.random.default_rng(seed)
    rows = sorted(set(spikes) | {1, Skv // 2} | set(int(x) for x in rng.integers(0, Skv, 64)))
    got_dv = to_f64(dv[0, 0, rows])
    got_dk = to_f64(dk[0, 0, rows])
    ref_dv = np.zeros((len(rows), d))
    ref_dk = np.zeros((len(rows), d))
    for i, j in enumerate(rows):
        pj = p.get(j, p_rest)
        vj = to_f64(v[0, 0, j])
        ref_dv[i] = pj * dof
        ref_dk[i] = scale * pj * (float(dof @ vj) - Dd) * qf
    ref_dq = scale * sum(p[j] * (float(dof @ vs[j]) - Dd) * ks[j] for j in spikes)
    assert_close(got_dv, ref_dv, TOL_GRAD, f"max-size bwd fused={fused} dV rows")
    assert_close(got_dk, ref_dk, TOL_GRAD, f"max-size bwd fused={fused} dK rows")
    assert_close(to_f64(dq)[0, 0, 0], ref_dq, TOL_GRAD, f"max-size bwd fused={fused} dQ")
    del q, do, k, v, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
