"""Benchmark of the online-softmax attention hot path on one MI355X.

One step = attn_fwd followed by attn_bwd on the training workload
(bf16, causal, B=4, H=16, S=2048, d=128): every row of the path except
split-KV decode, which is timed in the same run on its own workload
(bf16, B=8, Hq=32, Hkv=8, Skv=4096, d=128, 16 splits), as are the same
decode over a paged cache (shuffled 64-key pages), the training step with
a 512-key sliding window, the training step with an additive fp32 bias, the
fp32 128-token and bf16 transformer-block (S512 d64) forwards, and the
44k-token head-dim-256 causal prefill.  Inputs are seeded synthetic tensors already
resident in device memory; three input sets rotate so that no step reuses
the previous step's data from the 256 MiB last-level cache.

Prints one JSON line.  `value` = algorithmic TFLOP/s of the step (forward
4*d, backward 10*d FLOP per allowed (query, key) pair per head).  The
`roofline` object is for the kernel that takes the most time per step,
timed with HIP events recorded around that kernel inside the timed region.
`cpu_baseline` times the float64 oracle on a bounded sample on host cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--no-extras] [--only fwd_bwd|decode|paged_decode|prefill|small|tiles|gqa_bwd|fused_bwd]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention fwd/bwd TFLOP/s + % bf16 MFMA peak; decode HBM GB/s + % peak"

# Kernel names as they appear in a rocprofv3 kernel trace, per ABI call
# (the i-th kernel of each call, matching the timing-event slots).
KERNELS = {
    "fwd": ["fwd_bf16_kernel"],
    "bwd": ["bwd_dq_kernel", "bwd_dkdv_kernel"],
    "decode": ["decode_split_kernel", "decode_combine_kernel"],
}
# Steps of the per-kernel breakdown pass that precedes the timed region.
BREAKDOWN_STEPS = 100

SOURCES = {"fwd_bf16_kernel": "fwd.hip",
           "bwd_dkdv_kernel": "bwd_kernels.h", "bwd_dq_kernel": "bwd_kernels.h",
           "bwd_dkdv_fused_kernel": "bwd_kernels.h",
           "decode_split_kernel": "decode.hip", "decode_combine_kernel": "decode.hip"}


class HipEvents:
    """Timing events: torch's HIP events (the process's one HIP runtime),
    handed to the library by their raw hipEvent_t handles."""

    def __init__(self):
        self.made = []

    def create(self, n):
        import torch
        out = []
        for _ in range(n):
            e = torch.cuda.Event(enable_timing=True)
            e.record()  # creates the underlying hipEvent_t
            out.append(e)
        torch.cuda.synchronize()
        for e in out:
            if not e.cuda_event:
                raise RuntimeError("could not create a HIP event")
        self.made += out
        return out

    @staticmethod
    def handles(events):
        return [e.cuda_event for e in events]

    @staticmethod
    def record(ev, stream):
        ev.record(stream)

    @staticmethod
    def ms(a, b):
        return a.elapsed_time(b)

    def destroy(self):
        self.made = []


def flops_fwd(w):
    return 4.0 * w.d * w.pairs_per_head() * w.B * w.Hq


def per_kernel_algorithmic(w):
    """Algorithmic work per launch of each kernel: ("mfma", FLOP) or ("hbm", bytes)."""
    pairs = w.pairs_per_head() * w.B * w.Hq
    es = 2
    q_bytes = w.B * w.Hq * w.Sq * w.d * es
    kv_bytes = w.B * w.Hkv * w.Skv * w.d * es
    out = {
        # forward: Q K^T and P V, 2 FLOP per multiply-add each
        "fwd_bf16_kernel": ("mfma", 4.0 * w.d * pairs),
        # S, dP, dV and dK products (the recomputed S is one of the five
        # backward products, so it is credited here)
        "bwd_dkdv_kernel": ("mfma", 8.0 * w.d * pairs),
        # dQ product only; its recomputation of S and dP, and its D = rowsum(dO * O)
        # per query row, are not credited
        "bwd_dq_kernel": ("mfma", 2.0 * w.d * pairs),
    }
    if w.kind == "decode":
        split_bytes = 2 * kv_bytes + q_bytes + w.n_splits * w.B * w.Hq * (w.d + 2) * 4
        out = {"decode_split_kernel": ("hbm", float(split_bytes)),
               "decode_combine_kernel": ("hbm", float(w.n_splits * w.B * w.Hq * (w.d + 2) * 4
                                                      + q_bytes + w.B * w.Hq * 4))}
    return out


def source_hash(kernel):
    path = os.path.join(ROOT, "attention_online_softmax_amd", "csrc", SOURCES[kernel])
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "attention_online_softmax_amd", "csrc", "common.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current source of the kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(kernel):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return os.cpu_count() or 1


# Tolerances of the parity check on the timed inputs (max-abs against the
# float64 oracle), as in the parity tests.
TOL = {"O_bf16": 2e-2, "O_f32": 1e-5, "LSE_bf16": 1e-3, "LSE_f32": 1e-5, "grad": 5e-2}
PARITY_SLICES = 8   # (batch, head) slices of the timed step compared with the oracle


def _max_abs(a, b):
    import numpy as np
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if not np.all(np.isfinite(a)):
        return float("inf")
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def cpu_baseline(w, cpu_inputs, gpu_out=None, budget_s=15.0):
    """Time the oracle as it stands on whole heads of the same inputs (every
    (batch, head) in turn, starting over if all are done) until about
    budget_s seconds have passed; report algorithmic TFLOP/s.  The oracle's
    results for the first PARITY_SLICES slices are then compared (outside
    the timing) with the GPU's outputs of the timed step on those slices."""
    import oracle
    from attention_online_softmax_amd.inputs import to_f64
    q, k, v, do = (cpu_inputs[n] for n in ("q", "k", "v", "do"))
    G = w.Hq // w.Hkv
    pairs = w.pairs_per_head()
    done, flop = 0, 0.0
    kept = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        i = done % (w.B * w.Hq)
        b, h = divmod(i, w.Hq)
        kh = h // G
        qq = to_f64(q[b:b + 1, h:h + 1])
        kk = to_f64(k[b:b + 1, kh:kh + 1])
        vv = to_f64(v[b:b + 1, kh:kh + 1])
        dd = to_f64(do[b:b + 1, h:h + 1])
        O, lse = oracle.attention_ref(qq, kk, vv, w.causal, w.scale)
        grads = oracle.attention_bwd_ref(qq, kk, vv, dd, w.causal, w.scale, lse=lse)
        if done < PARITY_SLICES and G == 1:
            kept.append((b, h, O, lse, grads[:3]))
        done += 1
        flop += 14.0 * w.d * pairs
    dt = time.perf_counter() - t0
    parity = None
    if gpu_out is not None and kept:
        err = {"O": 0.0, "LSE": 0.0, "dQ": 0.0, "dK": 0.0, "dV": 0.0}
        for b, h, O, lse, (rq, rk, rv) in kept:
            sl = (slice(b, b + 1), slice(h, h + 1))
            for name, ref in (("O", O), ("dQ", rq), ("dK", rk), ("dV", rv)):
                key = {"O": "o", "dQ": "dq", "dK": "dk", "dV": "dv"}[name]
                err[name] = max(err[name], _max_abs(to_f64(gpu_out[key][sl]), ref))
            err["LSE"] = max(err["LSE"], _max_abs(gpu_out["lse"][sl].numpy(), lse))
        tol = {"O": TOL["O_bf16"], "LSE": TOL["LSE_bf16"], "dQ": TOL["grad"], "dK": TOL["grad"],
               "dV": TOL["grad"]}
        parity = {"slices": [[b, h] for b, h, *_ in kept], "max_abs": err, "tol": tol,
                  "pass": all(err[x] <= tol[x] for x in err)}
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
            "cores_meaning": "BLAS threads of numpy's matrix products (the element-wise "
                             "exp runs on one thread)",
            "host_affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"float64 oracle forward+backward on {done} (batch, head) slices of the "
                      f"same inputs ({w.B * w.Hq} distinct, taken in order), full S={w.Sq}, "
                      f"{dt:.1f} s",
            "seconds": dt, "parity_on_timed_inputs": parity}


def parity_extras(extras, probes):
    """The other timed workloads' outputs (first input set) against the
    oracle: the decode and paged decode in full, the small forwards in full,
    the 44k prefill on 16 rows of every head (first 8 and last 8)."""
    import numpy as np
    import oracle
    from attention_online_softmax_amd.inputs import to_f64
    out = {}
    if "decode" in probes:
        w, cpu, o, lse = probes["decode"]
        O, L = oracle.decode_ref(to_f64(cpu["q"]), to_f64(cpu["k"]), to_f64(cpu["v"]), w.scale,
                                 w.n_splits)
        out["decode"] = {"O": _max_abs(to_f64(o), O), "LSE": _max_abs(lse.numpy(), L),
                         "tol": {"O": TOL["O_bf16"], "LSE": TOL["LSE_bf16"]}}
    if "paged_decode" in probes:
        cpu, scale, o, lse = probes["paged_decode"]
        ref = {k: (to_f64(v) if v.is_floating_point() else v.numpy()) for k, v in cpu.items()}
        O, L = oracle.decode_paged_ref(ref["q"], ref["k_pages"], ref["v_pages"], ref["block_table"],
                                       ref["seq_lens"], scale)
        out["paged_decode"] = {"O": _max_abs(to_f64(o), O), "LSE": _max_abs(lse.numpy(), L),
                               "tol": {"O": TOL["O_bf16"], "LSE": TOL["LSE_bf16"]}}
    for key in ("fp32_small", "block_fwd"):
        if key in probes:
            w, cpu, o, lse = probes[key]
            O, L = oracle.attention_ref(to_f64(cpu["q"]), to_f64(cpu["k"]), to_f64(cpu["v"]),
                                        w.causal, w.scale)
            out[key] = {"O": _max_abs(to_f64(o), O), "LSE": _max_abs(lse.numpy(), L),
                        "tol": {"O": TOL[f"O_{w.dtype}"], "LSE": TOL[f"LSE_{w.dtype}"]}}
    if "long_prefill" in probes:
        w, cpu, rows, o, lse = probes["long_prefill"]
        O, L = oracle.attention_ref(to_f64(cpu["q"]), to_f64(cpu["k"]), to_f64(cpu["v"]), w.causal,
                                    w.scale, rows=np.asarray(rows))
        out["long_prefill"] = {"rows_per_head": len(rows), "O": _max_abs(to_f64(o), O),
                               "LSE": _max_abs(lse.numpy(), L),
                               "tol": {"O": TOL["O_bf16"], "LSE": TOL["LSE_bf16"]}}
    for r in out.values():
        r["pass"] = all(r[x] <= r["tol"][x] for x in r["tol"])
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def run_conditions():
    """What the numbers depend on besides the code: device, driver and
    toolchain versions, the build flags, the library that was timed and the
    host cores ("Compilers and Kernels", section "Operating the
    compiler-kernel boundary": pin architecture, runtime, toolchain and
    flags)."""
    import torch
    from attention_online_softmax_amd import build as B
    from attention_online_softmax_amd.binding import LIB_PATH
    props = torch.cuda.get_device_properties(0)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    try:
        with open(os.path.join(rocm, ".info", "version")) as f:
            rocm_version = f.read().strip()
    except OSError:
        rocm_version = None
    # The toolchain and flags come from the build's own record (no compiler
    # is started from this process); the library's hash is taken here.
    try:
        with open(B.BUILD_INFO) as f:
            info = json.load(f)
    except (OSError, ValueError):
        info = {}
    h = hashlib.sha256()
    with open(LIB_PATH, "rb") as f:
        h.update(f.read())
    lib_hash = h.hexdigest()[:16]
    return {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm_version,
            "hip_runtime": torch.version.hip, "torch": torch.__version__,
            "hipcc": info.get("hipcc"),
            "build_flags": info.get("build_flags"), "per_file_flags": info.get("per_file_flags"),
            "libattn_sha256_16": lib_hash,
            "build_info_matches_library": info.get("libattn_sha256_16") == lib_hash,
            "cpu_model": cpu_model(), "host_affinity_cores": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads()}


def quantiles(xs):
    s = sorted(xs)
    n = len(s)
    return {"median": s[n // 2], "p10": s[max(0, int(0.1 * n))], "p90": s[min(n - 1, int(0.9 * n))]}


def run_calls(calls, n_kernels, hev, steps, stream, slots=None):
    """Run `steps` iterations of the ABI calls with HIP events bound by the
    library to its kernel launches.  slots: {call: set of event slots to
    record} (slot 2i = start of kernel i, 2i+1 = its end); None records every
    slot.  The events ride on the launches themselves, so none of them adds a
    packet or a gap to the stream.
    Returns (total ms between events bracketing all steps,
    {call: [[ms of kernel i, or None] per step]},
    {call: [ms from first recorded slot to last recorded slot] per step})."""
    import torch
    import attention_online_softmax_amd as aos
    per = {}
    for name, _ in calls:
        nk = n_kernels[name]
        want = set(range(2 * nk)) if slots is None else slots.get(name, set())
        evs = []
        for _ in range(steps):
            evs.append([hev.create(1)[0] if j in want else None for j in range(2 * nk)])
        per[name] = evs
    start, end = hev.create(2)
    torch.cuda.synchronize()
    hev.record(start, stream)
    for s in range(steps):
        for name, fn in calls:
            aos.attn_set_timing_events([e.cuda_event if e is not None else 0 for e in per[name][s]])
            fn(s)
    aos.attn_set_timing_events(None)
    hev.record(end, stream)
    torch.cuda.synchronize()
    total = hev.ms(start, end)
    times, spans = {}, {}
    for name, _ in calls:
        nk = n_kernels[name]
        t_name, s_name = [], []
        for ev in per[name]:
            t_name.append([hev.ms(ev[2 * i], ev[2 * i + 1])
                           if ev[2 * i] is not None and ev[2 * i + 1] is not None else None
                           for i in range(nk)])
            rec = [e for e in ev if e is not None]
            s_name.append(hev.ms(rec[0], rec[-1]) if len(rec) >= 2 else None)
        times[name], spans[name] = t_name, s_name
    return total, times, spans


def kernel_stats(times, name, w):
    out = {}
    algo = per_kernel_algorithmic(w)
    for i, kname in enumerate(KERNELS[name]):
        ms = [t[i] for t in times[name] if t[i] is not None]
        if not ms:
            continue
        avg = sum(ms) / len(ms)
        bound, work = algo[kname]
        rate = work / (avg * 1e-3) / (1e12 if bound == "mfma" else 1e9)
        out[kname] = {"avg_us": avg * 1e3, **{k + "_us": v * 1e3 for k, v in quantiles(ms).items()},
                      "bound": bound,
                      "achieved": rate,
                      "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                      "frac": rate / (PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS),
                      "work_per_launch": work}
    return out


def bench_fwd_bwd(args, hev, stream):
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload
    w = WORKLOADS["train_fwd_bwd"]
    cpu0 = make_workload(w)
    sets = [{k: v.cuda() for k, v in cpu0.items()}]
    for i in (1, 2):
        sets.append({k: v.cuda() for k, v in make_workload(w, w.seed_base + 100 * i).items()})
    outs = []
    for s in sets:
        o = torch.empty_like(s["q"])
        lse = torch.empty((w.B, w.Hq, w.Sq), device="cuda", dtype=torch.float32)
        ws = torch.empty(aos.attn_bwd_workspace_bytes(w.B, w.Hq, w.Sq, w.d), device="cuda",
                         dtype=torch.uint8)
        outs.append(dict(o=o, lse=lse, dq=torch.empty_like(s["q"]), dk=torch.empty_like(s["k"]),
                         dv=torch.empty_like(s["v"]), ws=ws))

    def fwd(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w.scale, o=o["o"], lse=o["lse"])

    def bwd(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_bwd(s["q"], s["k"], s["v"], o["o"], s["do"], o["lse"], causal=True, scale=w.scale,
                     dq=o["dq"], dk=o["dk"], dv=o["dv"], workspace=o["ws"])

    calls = [("fwd", fwd), ("bwd", bwd)]
    nk = {"fwd": 1, "bwd": 2}
    # Cold start, kept apart from the kernel times: the first call of each
    # entry point in the process (host wall time to completion, and GPU time
    # between events around it; includes loading the kernels' code).
    torch.cuda.synchronize()
    first = {}
    for name, fn in calls:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        fn(0)
        e1.record()
        torch.cuda.synchronize()
        first[name] = {"host_wall_ms": (time.perf_counter() - t0) * 1e3,
                       "gpu_ms": e0.elapsed_time(e1)}
    for i in range(args.warmup):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()
    # Instrumented pass: every kernel bracketed, for the breakdown and to find
    # the kernel that takes the most time per step.  It runs BREAKDOWN_STEPS
    # steps (about 37 ms), which also leaves the GPU at its steady clocks when
    # the timed region starts: measured from an idle GPU, the first tens of
    # milliseconds of steps run about 5 % slower (0.352 against 0.334 ms per
    # step after 5 or 100 steps of warmup).
    _, times_i, _ = run_calls(calls, nk, hev, BREAKDOWN_STEPS, stream)
    ks = {}
    ks.update(kernel_stats(times_i, "fwd", w))
    ks.update(kernel_stats(times_i, "bwd", w))
    dom = max(ks, key=lambda k: ks[k]["avg_us"])
    dom_call = "fwd" if dom in KERNELS["fwd"] else "bwd"
    dom_idx = KERNELS[dom_call].index(dom)
    # Timed region: events only around the dominant kernel.
    total_ms, times, _ = run_calls(calls, nk, hev, args.steps, stream,
                                   slots={dom_call: {2 * dom_idx, 2 * dom_idx + 1}})
    dom_stats = kernel_stats(times, dom_call, w)[dom]
    flop_fwd = flops_fwd(w)
    flop_step = flop_fwd * 3.5
    ms_step = total_ms / args.steps
    fwd_ms = ks["fwd_bf16_kernel"]["avg_us"] * 1e-3
    bwd_ms = sum(ks[k]["avg_us"] for k in KERNELS["bwd"]) * 1e-3
    return w, cpu0, {
        "ms_per_step": ms_step,
        "value": flop_step / (ms_step * 1e-3) / 1e12,
        "fwd": {"ms": fwd_ms, "TFLOP/s": flop_fwd / (fwd_ms * 1e-3) / 1e12},
        "bwd": {"ms": bwd_ms, "TFLOP/s": 2.5 * flop_fwd / (bwd_ms * 1e-3) / 1e12},
        "kernels": ks,
        "kernels_steps": BREAKDOWN_STEPS,
        "first_call": first,
        "dominant": dom,
        "dominant_timed": dom_stats,
        "_probe": {k: outs[0][k].cpu() for k in ("o", "lse", "dq", "dk", "dv")},
        "seeds": {"Q,K,V,dO of input sets 0,1,2": [[b + j for j in range(4)] for b in
                                                     (w.seed_base, w.seed_base + 100,
                                                      w.seed_base + 200)]},
    }


def bench_decode(args, hev, stream, reps):
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload
    w = WORKLOADS["gqa_decode"]
    sets = [{k: v.cuda() for k, v in make_workload(w, w.seed_base + 100 * i).items()}
            for i in range(3)]
    ws = torch.empty(aos.attn_decode_workspace_bytes(w.B, w.Hq, w.d, w.n_splits), device="cuda",
                     dtype=torch.uint8)
    outs = [(torch.empty_like(s["q"]), torch.empty((w.B, w.Hq, 1), device="cuda",
                                                   dtype=torch.float32)) for s in sets]

    def dec(i):
        s, (o, lse) = sets[i % 3], outs[i % 3]
        aos.attn_decode(s["q"], s["k"], s["v"], scale=w.scale, n_splits=w.n_splits, o=o, lse=lse,
                        workspace=ws)

    for i in range(5):
        dec(i)
    # Per-kernel breakdown (instrumented pass), then call spans with events
    # only before the first and after the last kernel.
    _, times, _ = run_calls([("decode", dec)], {"decode": 2}, hev, min(reps, 20), stream)
    ks = kernel_stats(times, "decode", w)
    total_ms, _, spans = run_calls([("decode", dec)], {"decode": 2}, hev, reps, stream,
                                   slots={"decode": {0, 3}})
    per_call = spans["decode"]
    q = quantiles(per_call)
    kv = 2.0 * w.B * w.Hkv * w.Skv * w.d * 2
    algo = kv + 2.0 * w.B * w.Hq * w.d * 2 + w.B * w.Hq * 4
    torch.cuda.synchronize()
    probe = (w, make_workload(w, w.seed_base), outs[0][0].cpu(), outs[0][1].cpu())
    return {"_probe": probe, "seeds": [w.seed_base + 100 * i for i in range(3)],
            "workload": "gqa_decode: bf16, B8 Hq32 Hkv8 Skv4096 d128, 16 splits",
            "us_median": q["median"] * 1e3, "us_p10": q["p10"] * 1e3, "us_p90": q["p90"] * 1e3,
            "us_per_call_issued_back_to_back": total_ms / reps * 1e3,
            "GB/s": algo / (q["median"] * 1e-3) / 1e9,
            "frac_of_8TBs": algo / (q["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes": algo, "kernels": ks}


def bench_decode_paged(args, hev, stream, reps):
    """The paged, variable-length decode at the grouped-query decode shape
    (same streams and bytes as gqa_decode, keys in shuffled 64-key pages)."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import PAGED_WORKLOAD as w, make_paged
    sets = [{k: v.cuda() for k, v in make_paged(w["B"], w["Hq"], w["Hkv"], w["d"], w["page_size"],
                                                 w["max_pages"], w["lens"],
                                                 seed=w["seed"] + 100 * i).items()}
            for i in range(3)]
    ws = torch.empty(aos.attn_decode_workspace_bytes(w["B"], w["Hq"], w["d"], w["n_splits"]),
                     device="cuda", dtype=torch.uint8)
    outs = [(torch.empty_like(s["q"]), torch.empty((w["B"], w["Hq"], 1), device="cuda",
                                                   dtype=torch.float32)) for s in sets]
    scale = 1.0 / math.sqrt(w["d"])

    def dec(i):
        s, (o, lse) = sets[i % 3], outs[i % 3]
        aos.attn_decode_paged(s["q"], s["k_pages"], s["v_pages"], s["block_table"], s["seq_lens"],
                              scale=scale, n_splits=w["n_splits"], o=o, lse=lse, workspace=ws)

    for i in range(5):
        dec(i)
    total_ms, _, spans = run_calls([("decode", dec)], {"decode": 2}, hev, reps, stream,
                                   slots={"decode": {0, 3}})
    q = quantiles(spans["decode"])
    keys = sum(w["lens"])
    algo = (2.0 * keys * w["Hkv"] * w["d"] * 2 + 2.0 * w["B"] * w["Hq"] * w["d"] * 2
            + w["B"] * w["Hq"] * 4 + w["B"] * (w["max_pages"] + 1) * 4)
    torch.cuda.synchronize()
    probe = (make_paged(w["B"], w["Hq"], w["Hkv"], w["d"], w["page_size"], w["max_pages"],
                        w["lens"], seed=w["seed"]), scale, outs[0][0].cpu(), outs[0][1].cpu())
    return {"_probe": probe, "seeds": [w["seed"] + 100 * i for i in range(3)],
            "workload": "paged_decode: bf16, B8 Hq32 Hkv8 d128, 4096 keys per stream in "
                        "shuffled 64-key pages, 16 splits",
            "us_median": q["median"] * 1e3, "us_p10": q["p10"] * 1e3, "us_p90": q["p90"] * 1e3,
            "us_per_call_issued_back_to_back": total_ms / reps * 1e3,
            "GB/s": algo / (q["median"] * 1e-3) / 1e9,
            "frac_of_8TBs": algo / (q["median"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "algorithmic_bytes": algo}


def bench_masked(args, hev, stream, reps, window=0, with_bias=False):
    """Forward + backward of the training shape (B4 H16 S2048 d128, causal)
    with a sliding window of `window` keys and/or an additive fp32 bias
    shared by all batches and heads ([1, 1, S, S], N(0, 1) values).
    Algorithmic FLOPs count the allowed pairs only (4 d per pair forward,
    10 d backward)."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload, randn
    w = WORKLOADS["train_fwd_bwd"]
    sets = [{k: v.cuda() for k, v in make_workload(w, w.seed_base + 100 * i).items()}
            for i in range(3)]
    bias = (randn((1, 1, w.Sq, w.Skv), w.seed_base + 7, 1.0, torch.float32).cuda()
            if with_bias else None)
    outs = []
    for s in sets:
        outs.append(dict(o=torch.empty_like(s["q"]),
                         lse=torch.empty((w.B, w.Hq, w.Sq), device="cuda", dtype=torch.float32),
                         dq=torch.empty_like(s["q"]), dk=torch.empty_like(s["k"]),
                         dv=torch.empty_like(s["v"]),
                         ws=torch.empty(aos.attn_bwd_workspace_bytes(w.B, w.Hq, w.Sq, w.d),
                                        device="cuda", dtype=torch.uint8)))

    def fwd(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w.scale, o=o["o"], lse=o["lse"],
                     window=window, bias=bias)

    def bwd(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_bwd(s["q"], s["k"], s["v"], o["o"], s["do"], o["lse"], causal=True, scale=w.scale,
                     dq=o["dq"], dk=o["dk"], dv=o["dv"], workspace=o["ws"], window=window,
                     bias=bias)

    for i in range(3):
        fwd(i)
        bwd(i)
    torch.cuda.synchronize()
    total_ms, _, spans = run_calls([("fwd", fwd), ("bwd", bwd)], {"fwd": 1, "bwd": 2}, hev, reps,
                                   stream, slots={"fwd": {0, 1}, "bwd": {0, 3}})
    off = w.Skv - w.Sq
    lo = (lambda i: max(0, i + off - window + 1)) if window > 0 else (lambda i: 0)
    pairs = sum(min(i + off + 1, w.Skv) - lo(i) for i in range(w.Sq))
    flop_fwd = 4.0 * w.d * pairs * w.B * w.Hq
    fq = quantiles([t for t in spans["fwd"] if t is not None])
    bq = quantiles([t for t in spans["bwd"] if t is not None])
    ms = total_ms / reps
    what = ", ".join(x for x in (f"window {window}" if window > 0 else "",
                                 "shared fp32 bias [1,1,S,S]" if with_bias else "") if x)
    return {"workload": f"train shape bf16 causal B4 H16 S2048 d128, {what}",
            "ms_per_step": ms, "TFLOP/s": 3.5 * flop_fwd / (ms * 1e-3) / 1e12,
            "fwd_ms": fq["median"], "fwd_TFLOP/s": flop_fwd / (fq["median"] * 1e-3) / 1e12,
            "bwd_ms": bq["median"], "bwd_TFLOP/s": 2.5 * flop_fwd / (bq["median"] * 1e-3) / 1e12,
            "frac_of_bf16_peak": 3.5 * flop_fwd / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def bench_fused_bwd(args, hev, stream, reps):
    """Backward of the training shape (B4 H16 S2048 d128, causal) two ways:
    the two-kernel attn_bwd (dQ kernel, then dK/dV) and attn_bwd_fused (one
    pass over the key tiles, dQ added with fp32 atomics).  Reports the call
    times, the fused call's kernels and the bytes its atomics add."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload
    w = WORKLOADS["train_fwd_bwd"]
    sets = [{k: v.cuda() for k, v in make_workload(w, w.seed_base + 100 * i).items()}
            for i in range(3)]
    outs = []
    for s in sets:
        o, lse = aos.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w.scale)
        outs.append(dict(o=o, lse=lse, dq=torch.empty_like(s["q"]), dk=torch.empty_like(s["k"]),
                         dv=torch.empty_like(s["v"]),
                         ws=torch.empty(aos.attn_bwd_workspace_bytes(w.B, w.Hq, w.Sq, w.d),
                                        device="cuda", dtype=torch.uint8),
                         wsf=torch.empty(aos.attn_bwd_fused_workspace_bytes(w.B, w.Hq, w.Sq, w.d),
                                         device="cuda", dtype=torch.uint8)))

    def two(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_bwd(s["q"], s["k"], s["v"], o["o"], s["do"], o["lse"], causal=True, scale=w.scale,
                     dq=o["dq"], dk=o["dk"], dv=o["dv"], workspace=o["ws"])

    def fused(i):
        s, o = sets[i % 3], outs[i % 3]
        aos.attn_bwd_fused(s["q"], s["k"], s["v"], o["o"], s["do"], o["lse"], causal=True,
                           scale=w.scale, dq=o["dq"], dk=o["dk"], dv=o["dv"], workspace=o["wsf"])

    for i in range(3):
        two(i)
        fused(i)
    torch.cuda.synchronize()
    _, times, spans = run_calls([("two", two), ("fused", fused)], {"two": 2, "fused": 3}, hev,
                                reps, stream)
    tq = quantiles([t for t in spans["two"] if t is not None])
    fq = quantiles([t for t in spans["fused"] if t is not None])
    names = ("prep_kernel", "dkdv_dq_fused_kernel", "dq_convert_kernel")
    kern = {nm: quantiles([t[i] for t in times["fused"] if t[i] is not None])["median"] * 1e3
            for i, nm in enumerate(names)}
    # fp32 bytes added by the atomics: per (128-key tile, 32-query tile) pair
    # that the causal loop visits, min(32, Sq - q0) rows of d floats.
    off = w.Skv - w.Sq
    atom = 0
    for kt in range((w.Skv + 127) // 128):
        q0 = max(0, kt * 128 - off) // 32 * 32
        for qs in range(q0, w.Sq, 32):
            atom += min(32, w.Sq - qs) * w.d * 4
    atom *= w.B * w.Hq
    flop_bwd = 2.5 * flops_fwd(w)
    return {"workload": "train shape bf16 causal B4 H16 S2048 d128, backward only",
            "two_kernel_us": tq["median"] * 1e3, "fused_us": fq["median"] * 1e3,
            "two_kernel_TFLOP/s": flop_bwd / (tq["median"] * 1e-3) / 1e12,
            "fused_TFLOP/s": flop_bwd / (fq["median"] * 1e-3) / 1e12,
            "fused_kernels_us": kern, "dq_atomic_bytes": atom,
            "dq_atomic_GB/s_over_fused_kernel": atom / (kern["dkdv_dq_fused_kernel"] * 1e-6) / 1e9}


def bench_gqa_bwd(args, hev, stream, reps):
    """Backward with grouped heads (eight query heads per key/value head),
    bf16 causal d128 S4096, on two grids smaller than the chip: B4 Hq32 Hkv4
    (512 128-key workgroups for dK/dV) and B1 Hq32 Hkv4 (128).  Times the
    library's launch shapes (wave groups, and the head split when the
    workspace it asks for holds partial sums: then a third kernel sums them)
    and, for comparison, both kernels forced to the plain (4, 1) shape
    without a split."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import make_qkv
    res = {"workload": "gqa_bwd: bf16 causal Hq32 Hkv4 S4096 d128, backward only, B4 and B1"}
    for B in (4, 1):
        Hq, Hkv, S, d = 32, 4, 4096, 128
        seed = 6000 + B
        x = {k: v.cuda() for k, v in make_qkv(B, Hq, Hkv, S, S, d, seed=seed,
                                               with_do=True).items()}
        scale = d ** -0.5
        o, lse = aos.attn_fwd(x["q"], x["k"], x["v"], causal=True, scale=scale)
        base_ws = aos.attn_bwd_workspace_bytes(B, Hq, S, d)
        split_ws = aos.attn_bwd_split_workspace_bytes(B, Hq, Hkv, S, S, d, True)
        g = dict(dq=torch.empty_like(x["q"]), dk=torch.empty_like(x["k"]),
                 dv=torch.empty_like(x["v"]),
                 ws=torch.empty(max(base_ws, split_ws), device="cuda", dtype=torch.uint8))

        def bwd(i):
            aos.attn_bwd(x["q"], x["k"], x["v"], o, x["do"], lse, causal=True, scale=scale,
                         dq=g["dq"], dk=g["dk"], dv=g["dv"], workspace=g["ws"])

        out = {"seed": seed}
        # the picked launch splits the heads when its workspace is the larger
        nk_picked = 3 if split_ws > base_ws else 2
        plan = aos.attn_bwd_plan(B, Hq, Hkv, S, S, d, True, workspace_bytes=max(base_ws, split_ws))
        assert (plan["hsplit"] > 1) == (nk_picked == 3)
        for name, shape, nk in (("picked", (0, 0, 0, 0, 0), nk_picked),
                                ("plain", (4, 1, 4, 1, 1), 2)):
            aos.attn_bwd_tile_override(*shape)
            try:
                for i in range(2):
                    bwd(i)
                torch.cuda.synchronize()
                _, times, spans = run_calls([("bwd", bwd)], {"bwd": nk}, hev, reps, stream)
            finally:
                aos.attn_bwd_tile_override(0, 0, 0, 0, 0)
            q = quantiles([t for t in spans["bwd"] if t is not None])
            kq = quantiles([t[0] for t in times["bwd"]])["median"]
            kk = quantiles([t[1] for t in times["bwd"]])["median"]
            flop = 10 * d * B * Hq * S * (S + 1) / 2   # 2.5 x the forward's 4 d per pair
            tf = flop / (q["median"] * 1e-3) / 1e12
            out[name] = {"us": q["median"] * 1e3, "dq_kernel_us": kq * 1e3,
                         "dkdv_kernel_us": kk * 1e3, "TFLOP/s": tf,
                         "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS}
            if nk == 3:
                out[name]["dkdv_reduce_kernel_us"] = quantiles([t[2] for t in times["bwd"]])["median"] * 1e3
            if name == "picked":
                out[name]["plan"] = {"dkdv": list(plan["dkdv"]), "dq": list(plan["dq"]),
                                     "hsplit": plan["hsplit"]}
        del x, o, lse, g
        res[f"B{B}"] = out
    return res


def measured_ceilings(stream):
    """What the box reaches, as the measured ceilings beside the spec peaks:
    HBM read bandwidth of a grid-stride streaming read of 1 GiB (three
    buffers rotate, so no pass is served by the 256 MiB last-level cache)
    and the bf16 matrix-core rate of 32x32x16 MFMAs fed from registers at two
    waves per SIMD (kernels in attention_online_softmax_amd/ceilings/)."""
    import ctypes
    import torch
    from attention_online_softmax_amd.build import CEIL_LIB
    L = ctypes.CDLL(CEIL_LIB)
    L.ceil_read_run.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p]
    L.ceil_mfma_run.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    st = ctypes.c_void_p(stream.cuda_stream)
    nbytes, blocks = 1 << 30, 1024
    bufs = [torch.ones(nbytes // 4, device="cuda", dtype=torch.int32) for _ in range(3)]
    out = torch.empty(blocks * 256, device="cuda", dtype=torch.float32)

    def read(i, nt=0):
        rc = L.ceil_read_run(ctypes.c_void_p(bufs[i % 3].data_ptr()), nbytes,
                             ctypes.c_void_p(out.data_ptr()), blocks, nt, st)
        if rc:
            raise RuntimeError(f"ceil_read_run: hip error {rc}")

    def timed(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    read_default = nbytes / timed(read, 12) / 1e9
    read_nt = nbytes / timed(lambda i: read(i, 1), 12) / 1e9
    read_gbs = max(read_default, read_nt)
    del bufs
    mblocks, iters = 512, 4000

    def mf(i):
        rc = L.ceil_mfma_run(ctypes.c_void_p(out.data_ptr()), mblocks, iters, st)
        if rc:
            raise RuntimeError(f"ceil_mfma_run: hip error {rc}")

    mfma_tf = mblocks * 4 * iters * 16 * 32768.0 / timed(mf, 5) / 1e12
    return {"hbm_read_GB/s": read_gbs,
            "hbm_read_kind": "grid-stride 16-byte loads over 1 GiB, 3 rotating buffers; "
                             "the faster of plain and non-temporal loads",
            "hbm_read_plain_GB/s": read_default, "hbm_read_nontemporal_GB/s": read_nt,
            "bf16_mfma_TFLOP/s": mfma_tf,
            "bf16_mfma_kind": "32x32x16 bf16 MFMAs from registers, 4 chains, 2 waves/SIMD",
            "spec_hbm_GB/s": PEAK_HBM_GBS, "spec_bf16_TFLOP/s": PEAK_BF16_TFLOPS}


def bench_small(args, hev, stream, reps):
    """The two small forward workloads: fp32 B1 H1 S128 d64 (non-causal) and the
    bf16 causal transformer-block forward B4 H16 S512 d64.  Cold: a 512 MiB
    fill runs before every call (outside the timed span), so the inputs come
    from HBM, not the 256 MiB last-level cache; warm: calls back to back on
    the same inputs.  Events bracket only the forward kernel."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    out = {}
    for key in ("fp32_small", "block_fwd"):
        w = WORKLOADS[key]
        s = {k: v.cuda() for k, v in make_workload(w).items()}
        o = torch.empty_like(s["q"])
        lse = torch.empty((w.B, w.Hq, w.Sq), device="cuda", dtype=torch.float32)

        def fwd(i):
            aos.attn_fwd(s["q"], s["k"], s["v"], causal=w.causal, scale=w.scale, o=o, lse=lse)

        def evict(i):
            flush.fill_(i & 255)

        fwd(0)
        torch.cuda.synchronize()
        res = {}
        for tag, calls in (("cold", [("evict", evict), ("fwd", fwd)]), ("warm", [("fwd", fwd)])):
            _, times, _ = run_calls(calls, {"evict": 0, "fwd": 1}, hev, reps, stream)
            res[tag] = quantiles([t[0] for t in times["fwd"] if t[0] is not None])
        es = 4 if w.dtype == "f32" else 2
        flop = flops_fwd(w)
        # Q, K, V read once; O and LSE written once
        nbytes = (2.0 * w.B * w.Hq * w.Sq * w.d * es + 2.0 * w.B * w.Hkv * w.Skv * w.d * es
                  + w.B * w.Hq * w.Sq * 4)
        peak_f = (157.3 if w.dtype == "f32" else PEAK_BF16_TFLOPS) * 1e12
        floor_us = max(flop / peak_f, nbytes / (PEAK_HBM_GBS * 1e9)) * 1e6
        torch.cuda.synchronize()
        r = {"_probe": (w, make_workload(w), o.cpu(), lse.cpu()), "seed": w.seed_base,
             "workload": f"{key}: {w.title}", "dtype": w.dtype,
             "us_median": res["cold"]["median"] * 1e3, "us_p10": res["cold"]["p10"] * 1e3,
             "us_p90": res["cold"]["p90"] * 1e3, "us_median_warm": res["warm"]["median"] * 1e3,
             "FLOP": flop, "algorithmic_bytes": nbytes,
             "roofline_floor_us": floor_us,
             "roofline_bound": "hbm" if nbytes / (PEAK_HBM_GBS * 1e9) > flop / peak_f else "mfma",
             "frac_of_roofline": floor_us / (res["cold"]["median"] * 1e3)}
        if w.dtype == "bf16":
            r["TFLOP/s"] = flop / (res["cold"]["median"] * 1e-3) / 1e12
            r["frac_of_bf16_peak"] = r["TFLOP/s"] / PEAK_BF16_TFLOPS
            r["GB/s"] = nbytes / (res["cold"]["median"] * 1e-3) / 1e9
            r["frac_of_8TBs"] = r["GB/s"] / PEAK_HBM_GBS
        out[key] = r
    return out


# Shapes of the tile-selection leg: (B, Hq, Hkv, S, d, causal).  The
# estimate's constants were calibrated on the first set; the second set was
# not used for that and validates the picks.
TILE_SHAPES_CAL = [
    (4, 16, 16, 2048, 128, True),    # the training forward
    (4, 16, 16, 512, 64, True),      # the transformer-block forward
    (1, 16, 2, 44032, 256, True),    # the 44k-token prefill
    (4, 16, 16, 1024, 64, True),
    (4, 16, 16, 512, 128, True),
    (1, 16, 16, 8192, 128, True),
    (8, 16, 16, 1024, 128, False),
    (4, 32, 4, 4096, 128, True),
    (2, 16, 16, 4096, 64, False),
    (16, 16, 16, 2048, 128, True),
    (2, 16, 2, 16384, 256, True),
    (1, 8, 8, 256, 128, False),
]
TILE_SHAPES_VAL = [
    (2, 32, 8, 3072, 128, True),
    (1, 32, 32, 4096, 64, True),
    (8, 8, 8, 768, 128, True),
    (4, 16, 4, 1536, 128, False),
    (1, 16, 2, 8192, 256, True),
    (2, 24, 24, 2048, 64, True),
    (16, 16, 16, 512, 128, True),
    (1, 64, 8, 6144, 128, True),
    (1, 8, 2, 512, 64, True),
]


def bench_tile_selection(args, hev, stream, reps=10):
    """Every compiled (waves per workgroup, keys per tile) candidate of the
    bf16 forward timed on each shape (warm, median of `reps` calls, events
    around the kernel), next to the per-tile estimate and the candidate it
    picks ("Tang", Abstract: the estimate picks the tile)."""
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import make_qkv
    rows = []
    for (B, Hq, Hkv, S, d, causal), role in ([(x, "calibration") for x in TILE_SHAPES_CAL]
                                            + [(x, "validation") for x in TILE_SHAPES_VAL]):
        x = {k: v.cuda() for k, v in make_qkv(B, Hq, Hkv, S, S, d, seed=777).items()}
        o = torch.empty_like(x["q"])
        lse = torch.empty((B, Hq, S), device="cuda", dtype=torch.float32)
        pick, cands = aos.attn_fwd_tile_plan(d, causal, B, Hq, Hkv, S, S)
        n_reps = reps if S < 16384 else max(3, reps // 3)
        for c in cands:
            aos.attn_fwd_tile_override(c["nw"], c["bc"], c["split"])

            def fwd(i):
                aos.attn_fwd(x["q"], x["k"], x["v"], causal=causal, scale=d ** -0.5, o=o, lse=lse)

            try:
                fwd(0)
                fwd(0)
                torch.cuda.synchronize()
                _, times, _ = run_calls([("fwd", fwd)], {"fwd": 1}, hev, n_reps, stream)
            finally:
                aos.attn_fwd_tile_override(0, 0)
            c["measured_us"] = quantiles([t[0] for t in times["fwd"] if t[0] is not None])[
                "median"] * 1e3
        fastest = min(range(len(cands)), key=lambda i: cands[i]["measured_us"])
        rows.append({"shape": f"B{B} Hq{Hq} Hkv{Hkv} S{S} d{d} {'causal' if causal else 'full'}",
                     "role": role,
                     "candidates": cands,
                     "pick": [cands[pick][k] for k in ("nw", "bc", "split")],
                     "fastest": [cands[fastest][k] for k in ("nw", "bc", "split")],
                     "pick_over_fastest": cands[pick]["measured_us"] / cands[fastest]["measured_us"]})
        print(f"[bench] tiles {rows[-1]['shape']}: pick {rows[-1]['pick']} "
              f"{rows[-1]['pick_over_fastest']:.3f}x fastest {rows[-1]['fastest']}",
              file=sys.stderr, flush=True)
    out = {"shapes": rows}
    for role in ("calibration", "validation"):
        rr = [r for r in rows if r["role"] == role]
        out[role] = {"picks_within_3pct": sum(r["pick_over_fastest"] <= 1.03 for r in rr),
                     "n_shapes": len(rr),
                     "worst_pick_over_fastest": max(r["pick_over_fastest"] for r in rr),
                     "mean_pick_over_fastest": sum(r["pick_over_fastest"] for r in rr) / len(rr)}
    out["picks_within_3pct"] = sum(r["pick_over_fastest"] <= 1.03 for r in rows)
    out["n_shapes"] = len(rows)
    return out


def bench_prefill(args, hev, stream, reps):
    import torch
    import attention_online_softmax_amd as aos
    from attention_online_softmax_amd.inputs import WORKLOADS, make_workload
    w = WORKLOADS["long_prefill"]
    s = {k: v.cuda() for k, v in make_workload(w).items()}
    o = torch.empty_like(s["q"])
    lse = torch.empty((w.B, w.Hq, w.Sq), device="cuda", dtype=torch.float32)

    def fwd(i):
        aos.attn_fwd(s["q"], s["k"], s["v"], causal=True, scale=w.scale, o=o, lse=lse)

    fwd(0)
    torch.cuda.synchronize()
    total_ms, times, _ = run_calls([("fwd", fwd)], {"fwd": 1}, hev, reps, stream)
    ms = [t[0] for t in times["fwd"] if t[0] is not None]
    q = quantiles(ms)
    fl = flops_fwd(w)
    torch.cuda.synchronize()
    rows = list(range(8)) + list(range(w.Sq - 8, w.Sq))
    idx = torch.tensor(rows, device="cuda")
    probe = (w, make_workload(w), rows, o[:, :, idx].cpu(), lse[:, :, idx].cpu())
    return {"_probe": probe, "seed": w.seed_base,
            "workload": "long_prefill: bf16 causal, B1 Hq16 Hkv2 S44032 d256",
            "ms_median": q["median"], "ms_p10": q["p10"], "ms_p90": q["p90"],
            "TFLOP/s": fl / (q["median"] * 1e-3) / 1e12,
            "frac_of_bf16_peak": fl / (q["median"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--only", choices=["fwd_bwd", "decode", "paged_decode", "prefill", "small",
                                       "tiles", "gqa_bwd", "fused_bwd"], default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_online_softmax_amd as aos
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    aos.lib()
    hev = HipEvents()
    stream = torch.cuda.current_stream()

    def strip(d):
        if isinstance(d, dict):
            return {k: strip(v) for k, v in d.items() if k != "_probe"}
        return d

    if args.only == "decode":
        print(json.dumps(strip(bench_decode(args, hev, stream, args.steps))), flush=True)
        return
    if args.only == "paged_decode":
        print(json.dumps(strip(bench_decode_paged(args, hev, stream, args.steps))), flush=True)
        return
    if args.only == "small":
        print(json.dumps(strip(bench_small(args, hev, stream, args.steps))), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps(strip(bench_prefill(args, hev, stream, args.steps))), flush=True)
        return
    if args.only == "tiles":
        print(json.dumps(bench_tile_selection(args, hev, stream)), flush=True)
        return
    if args.only == "gqa_bwd":
        print(json.dumps(bench_gqa_bwd(args, hev, stream, args.steps)), flush=True)
        return
    if args.only == "fused_bwd":
        print(json.dumps(strip(bench_fused_bwd(args, hev, stream, args.steps))), flush=True)
        return

    w, cpu0, r = bench_fwd_bwd(args, hev, stream)
    print(f"[bench] fwd+bwd: {r['ms_per_step']:.3f} ms/step, {r['value']:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    extras = {}
    if not args.no_extras and args.only is None:
        extras["decode"] = bench_decode(args, hev, stream, max(args.steps, 50))
        print(f"[bench] decode: {extras['decode']['us_median']:.1f} us", file=sys.stderr,
              flush=True)
        extras["paged_decode"] = bench_decode_paged(args, hev, stream, max(args.steps, 50))
        print(f"[bench] paged decode: {extras['paged_decode']['us_median']:.1f} us",
              file=sys.stderr, flush=True)
        extras["window_fwd_bwd"] = bench_masked(args, hev, stream, max(args.steps, 20), window=512)
        print(f"[bench] window 512 fwd+bwd: {extras['window_fwd_bwd']['ms_per_step']:.3f} ms/step",
              file=sys.stderr, flush=True)
        extras["bias_fwd_bwd"] = bench_masked(args, hev, stream, max(args.steps, 20),
                                              with_bias=True)
        print(f"[bench] bias fwd+bwd: {extras['bias_fwd_bwd']['ms_per_step']:.3f} ms/step",
              file=sys.stderr, flush=True)
        extras["fused_bwd"] = bench_fused_bwd(args, hev, stream, max(args.steps, 20))
        print(f"[bench] backward two-kernel {extras['fused_bwd']['two_kernel_us']:.1f} us, "
              f"fused {extras['fused_bwd']['fused_us']:.1f} us", file=sys.stderr, flush=True)
        extras["gqa_bwd"] = bench_gqa_bwd(args, hev, stream, max(3, min(args.steps, 10)))
        print("[bench] grouped-head backward: " + ", ".join(
            f"B{b} {extras['gqa_bwd'][f'B{b}']['picked']['us']:.0f} us (plain shapes "
            f"{extras['gqa_bwd'][f'B{b}']['plain']['us']:.0f} us)" for b in (4, 1)),
            file=sys.stderr, flush=True)
        extras["small_fwd"] = bench_small(args, hev, stream, max(args.steps, 50))
        print(f"[bench] fp32 S128 fwd {extras['small_fwd']['fp32_small']['us_median']:.1f} us, "
              f"block fwd {extras['small_fwd']['block_fwd']['us_median']:.1f} us",
              file=sys.stderr, flush=True)
        extras["tile_selection"] = bench_tile_selection(args, hev, stream)
        print(f"[bench] tile selection: {extras['tile_selection']['picks_within_3pct']} of "
              f"{extras['tile_selection']['n_shapes']} picks within 3 % of the fastest",
              file=sys.stderr, flush=True)
        extras["long_prefill"] = bench_prefill(args, hev, stream, max(3, min(args.steps, 10)))
        print(f"[bench] long prefill: {extras['long_prefill']['ms_median']:.2f} ms",
              file=sys.stderr, flush=True)

    ks = r["kernels"]
    dom = r["dominant"]
    d = r["dominant_timed"]
    traffic = stored_traffic(dom, w.key)
    roofline = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"],
                "peak": PEAK_BF16_TFLOPS if d["bound"] == "mfma" else PEAK_HBM_GBS,
                "unit": d["unit"], "frac": d["frac"], "traffic": traffic,
                "avg_us": d["avg_us"], "work_per_launch": d["work_per_launch"]}
    probes = {}
    for key in ("decode", "paged_decode", "long_prefill"):
        if key in extras:
            probes[key] = extras[key].pop("_probe")
    if "small_fwd" in extras:
        for key, r_small in extras["small_fwd"].items():
            probes[key] = r_small.pop("_probe")
    gpu_out = r.pop("_probe")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, cpu0, gpu_out)
        print(f"[bench] cpu baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads",
              file=sys.stderr, flush=True)
        if probes:
            cpu["parity_other_workloads"] = parity_extras(extras, probes)
    line = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "train_fwd_bwd: attn_fwd + attn_bwd, bf16 storage, fp32 "
                               "accumulate, causal, B4 H16 S2048 d128",
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "seq_len": w.Sq, "head_dim": w.d,
                   "causal": True, "parallelism": "single GPU"},
        "frac_of_bf16_peak": r["value"] / PEAK_BF16_TFLOPS,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "fwd": r["fwd"],
        "bwd": r["bwd"],
        "kernels": ks,
        "kernels_steps": r["kernels_steps"],
        "first_call": r["first_call"],
        "seeds": r["seeds"],
        "run_conditions": run_conditions(),
    }
    line.update(extras)
    if not args.no_extras and args.only is None:
        c = measured_ceilings(stream)
        c["roofline_frac_of_measured"] = roofline["achieved"] / (
            c["bf16_mfma_TFLOP/s"] if roofline["bound"] == "mfma" else c["hbm_read_GB/s"])
        if "decode" in line:
            c["decode_frac_of_measured_read"] = line["decode"]["GB/s"] / c["hbm_read_GB/s"]
        if "paged_decode" in line:
            c["paged_decode_frac_of_measured_read"] = (line["paged_decode"]["GB/s"]
                                                       / c["hbm_read_GB/s"])
        if "long_prefill" in line:
            c["long_prefill_frac_of_measured_mfma"] = (line["long_prefill"]["TFLOP/s"]
                                                       / c["bf16_mfma_TFLOP/s"])
        line["measured_ceilings"] = c
        print(f"[bench] measured ceilings: read {c['hbm_read_GB/s']:.0f} GB/s, "
              f"bf16 MFMA {c['bf16_mfma_TFLOP/s']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    print(json.dumps(line), flush=True)
    hev.destroy()


if __name__ == "__main__":
    main()
