"""Seeded synthetic inputs for the attention forward pass.

This module only draws random numbers and applies each workload's value
transform; it contains none of attention's arithmetic.  Both the GPU path's
callers (tests, benchmark, smoke check) and the fp64 oracle receive the very
same host tensors from here.

Recipe (one per workload, seed = workload number):
  * ``g = torch.Generator('cpu').manual_seed(seed)``;
  * ``torch.randn(B, H, N, d, dtype=float32, generator=g)`` for Q, then K,
    then V, in that order -- i.i.d. N(0, 1), so that with scale = 1/sqrt(d)
    the scaled scores have unit variance (the variance argument of
    "Transformer Attention: A Mathematical Deep Dive", section "Why Scale by
    sqrt(d_k)");
  * the workload's transform in fp32: x0.1 on Q, K, V (wide-head fp32 case);
    or, for the long-context case, for each (b, h) in order,
    ``torch.randperm(N, generator=g)[:round(0.01 * N)]`` picks key rows that
    are multiplied by 8 (peaked softmax rows);
  * a round-to-nearest-even cast to the workload dtype (``.to(dtype)``).
The oracle reads the cast tensors, never the fp32 draws.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

_DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


@dataclass(frozen=True)
class Workload:
    """One attention-forward problem: shapes, dtype, mask, scale, transform."""
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str            # "fp32" | "bf16" | "fp16"
    causal: bool
    seed: int
    transform: str = ""   # "" | "x0.1" | "peaked_keys"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype]

    @property
    def flops(self) -> float:
        """4*B*H*N^2*d, halved for the causal mask (the metric's convention)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2.0 if self.causal else f

    def as_dict(self) -> dict:
        return {"workload": self.name, "B": self.B, "H": self.H, "N": self.N,
                "d": self.d, "dtype": self.dtype, "causal": self.causal,
                "scale": self.scale, "seed": self.seed,
                "transform": self.transform or "none"}


# The five workloads, numbered 1..5 (seed = number).
WORKLOADS = {
    1: Workload("single-head fp32 N128 d64", 1, 1, 128, 64, "fp32", False, 1),
    2: Workload("wide-head fp32 N1024 d1024 x0.1", 1, 1, 1024, 1024, "fp32", False, 2, "x0.1"),
    3: Workload("batched bf16 B4 H32 N2048 d64", 4, 32, 2048, 64, "bf16", False, 3),
    4: Workload("causal bf16 B2 H32 N8192 d128", 2, 32, 8192, 128, "bf16", True, 4),
    5: Workload("long-context causal bf16 B1 H32 N65536 d128 peaked-keys",
                1, 32, 65536, 128, "bf16", True, 5, "peaked_keys"),
}


def peaked_key_count(N: int) -> int:
    """Number of key rows per head scaled by 8 in the long-context workload."""
    return int(round(0.01 * N))


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             transform: str = ""):
    """Host (CPU) Q, K, V of shape [B, H, N, d] per the recipe above."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    q = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    k = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    v = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    if transform == "x0.1":
        q.mul_(0.1)
        k.mul_(0.1)
        v.mul_(0.1)
    elif transform == "peaked_keys":
        n_pk = peaked_key_count(N)
        for b in range(B):
            for h in range(H):
                idx = torch.randperm(N, generator=g)[:n_pk]
                k[b, h, idx, :] *= 8.0
    elif transform:
        raise ValueError(f"unknown transform {transform!r}")
    td = _DTYPES[dtype]
    if td != torch.float32:
        q, k, v = q.to(td), k.to(td), v.to(td)
    return q, k, v


def workload_inputs(w: Workload):
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.transform)


def peaked_key_rows(w: Workload):
    """The key indices the long-context transform scaled, per (b, h): it
    replays the generator's draws (no data is kept)."""
    if w.transform != "peaked_keys":
        return {}
    g = torch.Generator(device="cpu")
    g.manual_seed(int(w.seed))
    for _ in range(3):  # skip the Q, K, V draws
        torch.randn(w.B, w.H, w.N, w.d, dtype=torch.float32, generator=g)
    out = {}
    n_pk = peaked_key_count(w.N)
    for b in range(w.B):
        for h in range(w.H):
            out[(b, h)] = torch.randperm(w.N, generator=g)[:n_pk]
    return out


def make_dout(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """Host upstream gradient dL/dO [B, H, N, d]: i.i.d. N(0, 1) from its own
    generator seeded with `seed`, cast to `dtype` (round to nearest even)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    td = _DTYPES[dtype]
    return x.to(td) if td != torch.float32 else x


def make_normal_device(shape, dtype: str, seed: int, device="cuda"):
    """A seeded i.i.d. N(0, 1) tensor drawn on the device (torch's device
    generator), cast to `dtype` (round to nearest even): for inputs too large
    to draw on the host in reasonable time, e.g. key sequences of millions of
    rows.  The tests hand the same cast tensor (copied to the host) to the
    oracle."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(*shape, dtype=torch.float32, generator=g, device=device)
    td = _DTYPES[dtype]
    return x.to(td) if td != torch.float32 else x
