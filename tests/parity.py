"""Helpers for GPU-vs-oracle parity: tolerances, row sampling, error metrics."""
from __future__ import annotations

import numpy as np
import torch

import oracle

# Tolerances on |O_gpu - O_oracle| and |lse_gpu - lse_oracle| (all in fp64).
# bf16 and fp32 are the stated bounds of the workload definitions.  fp16 has
# three more mantissa bits than bf16, so the roundings of P and O -- the
# error of the 16-bit path -- are 8x finer, and its O bounds are bf16's
# divided by 8 (measured: fp16 errors run 8-9x below bf16's on the same
# shapes, max |dO| at most 1e-3); the lse bound is the fp32 statistics' own.
TOL = {
    torch.bfloat16: dict(max_o=2e-2, mean_o=2e-3, max_lse=1e-3),
    torch.float16: dict(max_o=2.5e-3, mean_o=2.5e-4, max_lse=1e-3),
    torch.float32: dict(max_o=1e-4, mean_o=1e-4, max_lse=1e-3),
}


# Gradient tolerances, relative to the largest element of the reference
# gradient tensor (its natural scale; see the derivation in the gradient
# tests).  fp16's are bf16's divided by 8, as for the forward: its roundings
# of P, dS and the outputs are 8x finer (measured over 72 gradient tensors,
# 4 shapes x 6 seeds: fp16 max 5.8e-4 and mean 4.0e-5 of the scale at worst,
# against bf16's 5.7e-3 and 3.2e-4).
TOL_BWD = {
    torch.bfloat16: dict(max_rel=2e-2, mean_rel=2e-3),
    torch.float16: dict(max_rel=2.5e-3, mean_rel=2.5e-4),
    torch.float32: dict(max_rel=1e-4, mean_rel=1e-5),
}


def sample_rows(B, H, N, seed, per_head_random=64, full_tile_heads=None, tile=128,
                extra=None, heads=None):
    """Stratified, seeded sample of flat row ids (b*H + h)*N + i.

    Per head: the first and last rows, both sides of the first tile boundary,
    the middle, `per_head_random` uniform rows, and -- for the heads in
    `full_tile_heads` (default: all) -- every row of one random query tile.
    `extra` maps (b, h) -> iterable of positions to add.  `heads` (default:
    all) restricts the sample to those (b, h).
    """
    rng = np.random.default_rng(seed)
    rows = []
    n_tiles = (N + tile - 1) // tile
    for b in range(B):
        for h in range(H):
            if heads is not None and (b, h) not in heads:
                continue
            base = (b * H + h) * N
            pos = {0, 1, tile - 1, tile, N // 2, N - 2, N - 1}
            pos.update(rng.integers(0, N, size=per_head_random).tolist())
            if full_tile_heads is None or (b, h) in full_tile_heads:
                t = int(rng.integers(0, n_tiles))
                pos.update(range(t * tile, min(N, (t + 1) * tile)))
            if extra and (b, h) in extra:
                pos.update(int(p) for p in extra[(b, h)])
            rows.extend(base + p for p in sorted(p for p in pos if 0 <= p < N))
    return np.array(rows, dtype=np.int64)


def compare(o_gpu, lse_gpu, q, k, v, scale, causal, rows=None, threads=0):
    """Oracle on the given rows (all if None) vs the GPU result; returns a dict
    of error statistics.  o_gpu, lse_gpu: device or host tensors."""
    B, H, N, d = q.shape
    o_ref, lse_ref = oracle.attn_rows(q, k, v, scale, causal, rows, threads)
    og = o_gpu.detach().to("cpu").double().reshape(B * H * N, d).numpy()
    lg = lse_gpu.detach().to("cpu").double().reshape(B * H * N).numpy()
    if rows is not None:
        og, lg = og[rows], lg[rows]
    do = np.abs(og - o_ref)
    dl = np.abs(lg - lse_ref)
    return dict(max_o=float(do.max()), mean_o=float(do.mean()), max_lse=float(dl.max()),
                rows=int(o_ref.shape[0]), finite=bool(np.isfinite(og).all() and np.isfinite(lg).all()))


def score_rounding_bound(q, k, scale):
    """Probabilistic bound on the error of fp32-accumulated scaled scores:
    sqrt(d) * 2^-24 * scale * max_ij sum_c |q_ic k_jc| (the worst case has d in
    place of sqrt(d)).  A score perturbation of at most E moves every softmax
    output by at most 2 * E * max|v| and the log-sum-exp by at most E."""
    qa, ka = q.double().abs(), k.double().abs()
    mag = (qa @ ka.transpose(-1, -2)).max().item()
    return q.shape[-1] ** 0.5 * 2.0 ** -24 * scale * mag


def check(stats, dtype, extra_o=0.0, extra_lse=0.0):
    """Assert the error statistics are within the dtype's bounds.  extra_o and
    extra_lse widen the per-element (max) bounds by a derived worst-case term;
    the mean bound is never widened: a per-element worst case says nothing
    about the average error."""
    tol = dict(TOL[dtype])
    tol["max_o"] += extra_o
    tol["max_lse"] += extra_lse
    assert stats["finite"], stats
    assert stats["max_o"] <= tol["max_o"], (stats, tol)
    assert stats["mean_o"] <= tol["mean_o"], (stats, tol)
    assert stats["max_lse"] <= tol["max_lse"], (stats, tol)
