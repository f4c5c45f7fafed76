"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random tensors of the right shapes; it holds none of
the attention arithmetic.  Each tensor has its own seed (Q = base, K = base+1,
V = base+2, dO = base+3) and is drawn as float32 N(0, 1) on the CPU with a
`torch.Generator`, multiplied by the workload's factor and rounded to the
workload's storage dtype (bf16 by round-to-nearest-even).  The same rounded
tensors go to the GPU and, upcast exactly to float64, to the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    key: str
    title: str
    kind: str            # "fwd", "decode" or "fwd+bwd"
    dtype: str           # "f32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    d: int
    causal: bool
    mult: float = 1.0
    n_splits: int = 0
    seed_base: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def pairs_per_head(self) -> int:
        """Number of allowed (query, key) pairs per head (diagonal included)."""
        if not self.causal:
            return self.Sq * self.Skv
        off = self.Skv - self.Sq
        return sum(min(i + off + 1, self.Skv) for i in range(self.Sq))


# The five workloads: a tiny fp32 check, a transformer-block forward, an
# 8B-class grouped-query decode, a 44k-token head-dim-256 prefill and a
# training-shape forward plus backward.
WORKLOADS = {
    "fp32_small": Workload("fp32_small", "fp32 forward B1 H1 S128 d64, non-causal",
                           "fwd", "f32", 1, 1, 1, 128, 128, 64, False, 1.0, seed_base=1000),
    "block_fwd": Workload("block_fwd", "bf16 causal forward B4 H16 S512 d64",
                          "fwd", "bf16", 4, 16, 16, 512, 512, 64, True, 0.5, seed_base=2000),
    "gqa_decode": Workload("gqa_decode", "bf16 GQA decode B8 Hq32 Hkv8 Skv4096 d128, 16 splits",
                           "decode", "bf16", 8, 32, 8, 1, 4096, 128, False, 1.0,
                           n_splits=16, seed_base=3000),
    "long_prefill": Workload("long_prefill", "bf16 causal prefill B1 Hq16 Hkv2 S44032 d256",
                             "fwd", "bf16", 1, 16, 2, 44032, 44032, 256, True, 0.5,
                             seed_base=4000),
    "train_fwd_bwd": Workload("train_fwd_bwd", "bf16 causal forward+backward B4 H16 S2048 d128",
                              "fwd+bwd", "bf16", 4, 16, 16, 2048, 2048, 128, True, 1.0,
                              seed_base=5000),
}


# Paged, variable-length decode at the grouped-query decode shape: the same
# 8 streams of 4096 keys (B8 Hq32 Hkv8 d128), kept in 64-key pages handed
# out in a seeded random order from a shared pool, 16 splits.
PAGED_WORKLOAD = dict(B=8, Hq=32, Hkv=8, d=128, page_size=64, max_pages=64, lens=[4096] * 8,
                      n_splits=16, seed=6000)


def randn(shape, seed, mult=1.0, dtype=torch.bfloat16):
    """float32 N(0,1) from a CPU generator seeded with `seed`, times `mult`,
    rounded to `dtype`."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if mult != 1.0:
        t.mul_(mult)
    return t.to(dtype)


def make_qkv(B, Hq, Hkv, Sq, Skv, d, dtype=torch.bfloat16, seed=0, mult=1.0, with_do=False):
    """Seeded Q [B,Hq,Sq,d], K and V [B,Hkv,Skv,d] (and dO [B,Hq,Sq,d])."""
    out = {
        "q": randn((B, Hq, Sq, d), seed, mult, dtype),
        "k": randn((B, Hkv, Skv, d), seed + 1, mult, dtype),
        "v": randn((B, Hkv, Skv, d), seed + 2, mult, dtype),
    }
    if with_do:
        out["do"] = randn((B, Hq, Sq, d), seed + 3, 1.0, dtype)
    return out


def make_paged(B, Hq, Hkv, d, page_size, max_pages, lens, n_pages=None, dtype=torch.bfloat16,
               seed=0, mult=1.0):
    """Seeded paged-decode inputs: q [B,Hq,1,d]; key and value pools
    [n_pages,Hkv,page_size,d] (default n_pages = B*max_pages + 3, so some
    pages are unused); a block table [B,max_pages] int32 that hands out
    distinct pool pages in a seeded random order; seq_lens [B] int32."""
    if n_pages is None:
        n_pages = B * max_pages + 3
    if n_pages < B * max_pages:
        raise ValueError("the pool must hold B * max_pages distinct pages")
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) + 4)
    table = torch.randperm(n_pages, generator=g)[:B * max_pages].to(torch.int32)
    return {
        "q": randn((B, Hq, 1, d), seed, mult, dtype),
        "k_pages": randn((n_pages, Hkv, page_size, d), seed + 1, mult, dtype),
        "v_pages": randn((n_pages, Hkv, page_size, d), seed + 2, mult, dtype),
        "block_table": table.reshape(B, max_pages).contiguous(),
        "seq_lens": torch.tensor(list(lens), dtype=torch.int32),
    }


def make_workload(w: Workload, seed_base=None):
    """Inputs for a named workload (CPU tensors in the workload's dtype)."""
    base = w.seed_base if seed_base is None else seed_base
    return make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.d, w.torch_dtype, base, w.mult,
                    with_do=(w.kind == "fwd+bwd"))


def to_f64(t):
    """Exact upcast of a CPU/GPU tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
