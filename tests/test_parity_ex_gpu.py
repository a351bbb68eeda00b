"""GPU parity for unequal query/key lengths and per-batch key padding:
fa_fwd_ex (through the C ABI) against the fp64 oracle's extension
(oracle_attn_rows_ex), element by element.

Shapes span several tiles with ragged tails in both directions (more queries
than keys and fewer), causal bottom-right alignment with rows that keep no
key, padded batches with 0, some and all keys valid, and counts outside
[0, Nk] (clamped).
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
DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def inputs(B, H, Nq, Nk, d, dt, seed):
    q, _, _ = make_qkv(B, H, Nq, d, dt, seed)
    _, k, v = make_qkv(B, H, Nk, d, dt, seed + 1)
    return q, k, v


def check(q, k, v, causal, k_len, dt, scale=None, split_keys=True):
    B, H, Nq, d = q.shape
    scale = 1 / math.sqrt(d) if scale is None else scale
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device="cuda")
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale, k_len=kl,
                          split_keys=split_keys)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attn_rows_ex(q, k, v, scale, causal, None, k_len)
    og = o.double().cpu().reshape(-1, d).numpy()
    lg = lse.double().cpu().reshape(-1).numpy()
    empty = np.isneginf(l_ref)
    # rows with no kept key: exactly O = 0 and lse = -inf
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty])), "empty rows"
    full = ~empty
    assert np.isfinite(og).all() and np.isfinite(lg[full]).all()
    if full.any():
        do = np.abs(og[full] - o_ref[full])
        stats = dict(max_o=float(do.max()), mean_o=float(do.mean()),
                     max_lse=float(np.abs(lg[full] - l_ref[full]).max()), finite=True,
                     rows=int(full.sum()))
        parity.check(stats, DT[dt])
    return int(empty.sum())


SHAPES = [(1, 300), (77, 300), (300, 77), (129, 1), (256, 1000), (200, 200)]
CASES = [(dt, d) for dt, dims in (("bf16", (64, 128)), ("fp16", (128,)), ("fp32", (64, 256)))
         for d in dims]


@pytest.mark.parametrize("dt,d", CASES)
@pytest.mark.parametrize("Nq,Nk", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths_match_oracle(dt, d, Nq, Nk, causal):
    q, k, v = inputs(2, 2, Nq, Nk, d, dt, 3000 + Nq + 7 * Nk + d)
    n_empty = check(q, k, v, causal, None, dt)
    if causal and Nq > Nk:
        assert n_empty == 2 * 2 * (Nq - Nk)


@pytest.mark.parametrize("dt,d", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_key_padding_matches_oracle(dt, d, causal):
    Nq, Nk = 190, 333
    q, k, v = inputs(4, 2, Nq, Nk, d, dt, 4000 + d + int(causal))
    # all keys, a ragged count, none, and fewer keys than queries
    check(q, k, v, causal, [333, 150, 0, 64], dt)


def test_out_of_range_counts_are_clamped():
    q, k, v = inputs(3, 1, 100, 130, 128, "bf16", 4500)
    kl = torch.tensor([-7, 500, 65], dtype=torch.int32, device="cuda")
    for causal in (False, True):
        o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal, k_len=kl)
        o2, l2 = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=causal,
                              k_len=torch.tensor([0, 130, 65], dtype=torch.int32, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, l2)


def test_padded_keys_are_never_read():
    """NaN in keys and values past a batch's count leaves the result finite
    and bitwise unchanged."""
    q, k, v = inputs(2, 2, 150, 260, 128, "bf16", 4600)
    kl = torch.tensor([260, 97], dtype=torch.int32, device="cuda")
    a = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=True, k_len=kl)
    k2, v2 = k.clone(), v.clone()
    k2[1, :, 97:] = float("nan")
    v2[1, :, 97:] = float("nan")
    b = fa.attention(q.cuda(), k2.cuda(), v2.cuda(), causal=True, k_len=kl)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("d", [64, 1024])
def test_fp32_key_split_with_unequal_lengths(d):
    """Small fp32 grids split keys over ranges; a range of a padded or causal
    row may hold no kept key, and a row may have none at all."""
    q, k, v = inputs(2, 1, 40, 700, d, "fp32", 4700 + d)
    assert fa.fa_fwd_ex_workspace_size(2, 1, 40, 700, d, 1, fa.FA_DTYPE_FP32) > 0
    for causal in (False, True):
        check(q, k, v, causal, [700, 0], "fp32")
        check(q, k, v, causal, [333, 12], "fp32", split_keys=False)


def test_long_unequal_causal_bf16_on_sampled_rows():
    """A decode-like block: 1024 new queries over 32768 cached keys, causal
    bottom-right, persistent d = 128 kernel; the oracle computes sampled rows."""
    B, H, Nq, Nk, d = 1, 8, 1024, 32768, 128
    q, k, v = inputs(B, H, Nq, Nk, d, "bf16", 4800)
    kl = torch.tensor([30000], dtype=torch.int32, device="cuda")
    o, lse = fa.attention(q.cuda(), k.cuda(), v.cuda(), causal=True, k_len=kl)
    torch.cuda.synchronize()
    rows = parity.sample_rows(B, H, Nq, seed=5, per_head_random=24, tile=256)
    o_ref, l_ref = oracle.attn_rows_ex(q, k, v, 1 / math.sqrt(d), True, rows, [30000])
    og = o.double().cpu().reshape(-1, d).numpy()[rows]
    lg = lse.double().cpu().reshape(-1).numpy()[rows]
    do = np.abs(og - o_ref)
    parity.check(dict(max_o=float(do.max()), mean_o=float(do.mean()),
                      max_lse=float(np.abs(lg - l_ref).max()), finite=bool(np.isfinite(og).all()),
                      rows=len(rows)), torch.bfloat16)
