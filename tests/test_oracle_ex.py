"""Pins of the oracle's unequal-length and key-padding extension
(oracle_attn_rows_ex), CPU only.

Each check ties the extension to something other than its own index rule: the
already-pinned equal-length oracle on derived problems (truncated keys, a
square causal problem with filler queries in front), garbage in padded keys,
closed forms, and a 40-digit decimal brute force.  The shapes follow the
ScaledDotProductAttention listing of "Transformer Attention: A Mathematical
Deep Dive": query (batch, n, d_k), key and value (batch, m, d), with a mask
"for causal attention or padding".
"""
import decimal

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_without_padding_is_the_plain_oracle(causal):
    q, k, v = (_rand((2, 3, 37, 8), s) for s in (1, 2, 3))
    o1, l1 = oracle.attention(q, k, v, 0.4, causal)
    o2, l2 = oracle.attention_ex(q, k, v, 0.4, causal)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_key_padding_equals_truncated_keys(causal):
    """Batch b with L valid keys gives what the problem with only its first L
    keys gives (for causal, aligned at the last valid key)."""
    B, H, Nq, Nk, d = 3, 2, 19, 41, 6
    q = _rand((B, H, Nq, d), 11)
    k, v = _rand((B, H, Nk, d), 12), _rand((B, H, Nk, d), 13)
    k_len = [41, 25, 7]
    o, lse = oracle.attention_ex(q, k, v, 0.5, causal, k_len)
    for b, L in enumerate(k_len):
        ot, lt = oracle.attention_ex(q[b:b + 1], k[b:b + 1, :, :L].contiguous(),
                                     v[b:b + 1, :, :L].contiguous(), 0.5, causal)
        assert np.array_equal(o[b:b + 1], ot) and np.array_equal(lse[b:b + 1], lt)


def test_padded_keys_are_never_read():
    B, H, Nq, Nk, d = 2, 2, 13, 30, 5
    q = _rand((B, H, Nq, d), 21)
    k, v = _rand((B, H, Nk, d), 22), _rand((B, H, Nk, d), 23)
    k_len = [30, 11]
    o, lse = oracle.attention_ex(q, k, v, 0.6, True, k_len)
    k2, v2 = k.clone(), v.clone()
    k2[1, :, 11:] = float("nan")
    v2[1, :, 11:] = 1e300
    o2, lse2 = oracle.attention_ex(q, k2, v2, 0.6, True, k_len)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_causal_short_query_block_is_the_end_of_a_square_problem():
    """Nq < Nk, causal: query i sits at position i + Nk - Nq of the keys, so the
    rows equal the last Nq rows of the square causal problem whose first
    Nk - Nq queries are arbitrary."""
    B, H, Nq, Nk, d = 1, 2, 9, 33, 7
    q = _rand((B, H, Nq, d), 31)
    k, v = _rand((B, H, Nk, d), 32), _rand((B, H, Nk, d), 33)
    o, lse = oracle.attention_ex(q, k, v, 0.45, True)
    qs = torch.cat([_rand((B, H, Nk - Nq, d), 34), q], dim=2)
    os_, ls = oracle.attention(qs, k, v, 0.45, True)
    assert np.array_equal(o, os_[:, :, Nk - Nq:]) and np.array_equal(lse, ls[:, :, Nk - Nq:])
    # the last query sees every key: the non-causal row
    onc, lnc = oracle.attention_ex(q, k, v, 0.45, False)
    assert np.abs(o[:, :, -1] - onc[:, :, -1]).max() < 1e-15


def test_causal_long_query_block_has_empty_leading_rows():
    """Nq > Nk, causal: the first Nq - Nk rows keep no key (o = 0, lse = -inf);
    the rest are the square causal problem of the last Nk queries."""
    B, H, Nq, Nk, d = 2, 1, 20, 8, 4
    q = _rand((B, H, Nq, d), 41)
    k, v = _rand((B, H, Nk, d), 42), _rand((B, H, Nk, d), 43)
    o, lse = oracle.attention_ex(q, k, v, 0.7, True)
    assert np.all(o[:, :, :Nq - Nk] == 0) and np.all(np.isneginf(lse[:, :, :Nq - Nk]))
    os_, ls = oracle.attention(q[:, :, Nq - Nk:].contiguous(), k, v, 0.7, True)
    assert np.array_equal(o[:, :, Nq - Nk:], os_) and np.array_equal(lse[:, :, Nq - Nk:], ls)


def test_no_valid_key_gives_the_empty_sum():
    q = _rand((2, 2, 5, 3), 51)
    k, v = _rand((2, 2, 6, 3), 52), _rand((2, 2, 6, 3), 53)
    for causal in (False, True):
        o, lse = oracle.attention_ex(q, k, v, 1.0, causal, [0, 6])
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
        assert np.all(np.isfinite(lse[1]))


def test_zero_queries_average_the_valid_values():
    B, H, Nq, Nk, d = 2, 3, 4, 10, 5
    q = torch.zeros(B, H, Nq, d, dtype=torch.float64)
    k, v = _rand((B, H, Nk, d), 61), _rand((B, H, Nk, d), 62)
    k_len = [10, 3]
    o, lse = oracle.attention_ex(q, k, v, 0.3, False, k_len)
    for b, L in enumerate(k_len):
        mean = v[b, :, :L].mean(dim=1, keepdim=True).numpy()
        assert np.abs(o[b] - mean).max() < 1e-14
        assert np.abs(lse[b] - np.log(L)).max() < 1e-14


def _decimal_row(qi, K, V, scale, kept):
    decimal.getcontext().prec = 40
    D = decimal.Decimal
    s = [D(scale) * sum(D(a) * D(b) for a, b in zip(qi, K[j])) for j in kept]
    m = max(s)
    e = [(x - m).exp() for x in s]
    tot = sum(e)
    o = [float(sum(e[t] * D(V[j][c]) for t, j in enumerate(kept)) / tot) for c in range(len(V[0]))]
    return o, float(m + tot.ln())


@pytest.mark.parametrize("Nq,Nk,L", [(3, 7, 7), (6, 4, 4), (5, 8, 6), (1, 5, 2)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(Nq, Nk, L, causal):
    d = 3
    q = _rand((1, 1, Nq, d), 70 + Nq)
    k, v = _rand((1, 1, Nk, d), 80 + Nk), _rand((1, 1, Nk, d), 90 + Nk)
    o, lse = oracle.attention_ex(q, k, v, 0.8, causal, [L])
    for i in range(Nq):
        kept = [j for j in range(L) if not causal or j <= i + L - Nq]
        if not kept:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
            continue
        ro, rl = _decimal_row(q[0, 0, i].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.8, kept)
        assert np.abs(o[0, 0, i] - ro).max() < 1e-12 and abs(lse[0, 0, i] - rl) < 1e-12


def test_invalid_shapes_are_rejected():
    q = _rand((1, 1, 4, 3), 99)
    with pytest.raises(ValueError):
        oracle.attn_rows_ex(q, q[..., :2].contiguous(), q[..., :2].contiguous(), 1.0, False)
    with pytest.raises(ValueError):
        oracle.attn_rows_ex(q, q, q, 1.0, False, k_len=[1, 2])
    with pytest.raises(ValueError):
        oracle.attn_rows_ex(q, q, q, 1.0, False, rows=[4])
