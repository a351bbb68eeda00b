"""Seeded sweep of the fp32 forward at the head dims split across waves
(d = 512: four waves of 128 columns, d = 1024: eight), against the fp64
oracle: ragged and unequal lengths, per-batch key and query counts, causal or
not, and grids small enough to take the key split as well as grids that do
not.  These shapes exercise the per-wave K slices loaded into LDS, the V rows
requested during the previous tile's products, the score exchange between the
waves and the staged output stores, each at a partial last tile.
Outputs start as NaN so that a row the kernel fails to write shows up.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_29_amd as fa
import oracle
from exact_attention_29_amd.inputs import make_qkv
from tests import parity

pytestmark = pytest.mark.gpu


def draw(i):
    """Case i: (B, H, Nq, Nk, d, causal, k_len, q_len, split)."""
    r = np.random.default_rng(7000 + i)
    d = [512, 1024][i % 2]
    B, H = int(r.integers(1, 3)), int(r.integers(1, 3))
    Nq, Nk = int(r.integers(1, 700)), int(r.integers(1, 700))
    causal = bool(r.integers(2))
    k_len = [int(x) for x in r.integers(0, Nk + 1, B)] if r.random() < 0.5 else None
    q_len = [int(x) for x in r.integers(0, Nq + 1, B)] if r.random() < 0.5 else None
    split = bool(r.integers(2))
    return B, H, Nq, Nk, d, causal, k_len, q_len, split


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("i", range(16))
def test_wide_fp32_case_matches_oracle(i):
    B, H, Nq, Nk, d, causal, k_len, q_len, split = draw(i)
    print("case", i, dict(B=B, H=H, Nq=Nq, Nk=Nk, d=d, causal=causal, k_len=k_len, q_len=q_len,
                          split=split), flush=True)
    q, k, _ = make_qkv(B, H, max(Nq, Nk), d, "fp32", 8000 + i)
    _, _, v = make_qkv(B, H, Nk, d, "fp32", 9000 + i)
    q, k = q[:, :, :Nq].contiguous(), k[:, :, :Nk].contiguous()
    scale = 1 / math.sqrt(d)
    dev = torch.device("cuda")
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device=dev)
    ql = None if q_len is None else torch.tensor(q_len, dtype=torch.int32, device=dev)
    o = torch.full((B, H, Nq, d), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, k_len=kl, q_len=ql,
                 split_keys=split, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_rows_ex(q, k, v, scale, causal, None, k_len, q_len=q_len)
    og = o.double().cpu().reshape(-1, d).numpy()
    lg = lse.double().cpu().reshape(-1).numpy()
    assert np.isfinite(og).all(), "an output row was not written"
    empty = np.isneginf(l_ref)
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty]))
    if (~empty).any():
        do = np.abs(og[~empty] - o_ref[~empty])
        parity.check(dict(max_o=float(do.max()), mean_o=float(do.mean()),
                          max_lse=float(np.abs(lg[~empty] - l_ref[~empty]).max()),
                          finite=True, rows=int((~empty).sum())), torch.float32)
