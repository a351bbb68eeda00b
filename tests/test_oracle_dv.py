"""Pins of the oracle's value head dim (oracle_attn_rows_gen and
oracle_attn_bwd_gen: Q and K of d_k columns, V, O and dO of d_v), CPU only.

The scaled dot-product attention of "Transformer Attention: A Mathematical
Deep Dive" takes Q of shape (n, d_k), K (m, d_k) and V (m, d_v).  Zero
columns change nothing: a zero column of V adds a zero column to O (and to
dV), and zero columns of Q and K add exact zeros to every score.  So each
problem with d_v != d_k is, bitwise, a problem of equal head dims -- the one
the plain oracles (pinned elsewhere) compute -- padded with zeros.  Beside
those reductions: a decimal brute force of tiny rows and central differences
of the forward for the gradients.
"""
import decimal

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _pad(x, width):
    """x with zero columns appended up to `width` head-dim columns."""
    out = torch.zeros(*x.shape[:3], width, dtype=x.dtype)
    out[..., : x.shape[3]] = x
    return out


SHAPES = [(2, 2, 9, 9, None), (2, 1, 5, 12, [12, 4]), (1, 2, 11, 6, None)]


@pytest.mark.parametrize("B,H,Nq,Nk,k_len", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_narrow_values_are_the_equal_dim_problem_with_zero_value_columns(B, H, Nq, Nk, k_len, causal):
    dk, dv = 7, 3
    q, k, v = _rand((B, H, Nq, dk), 1), _rand((B, H, Nk, dk), 2), _rand((B, H, Nk, dv), 3)
    o, lse = oracle.attention_ex(q, k, v, 0.6, causal, k_len)
    assert o.shape == (B, H, Nq, dv)
    op, lp = oracle.attention_ex(q, k, _pad(v, dk), 0.6, causal, k_len)
    assert np.array_equal(o, op[..., :dv]) and np.all(op[..., dv:] == 0)
    assert np.array_equal(lse, lp)


@pytest.mark.parametrize("B,H,Nq,Nk,k_len", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_wide_values_are_the_equal_dim_problem_with_zero_score_columns(B, H, Nq, Nk, k_len, causal):
    dk, dv = 3, 8
    q, k, v = _rand((B, H, Nq, dk), 4), _rand((B, H, Nk, dk), 5), _rand((B, H, Nk, dv), 6)
    o, lse = oracle.attention_ex(q, k, v, 0.9, causal, k_len)
    op, lp = oracle.attention_ex(_pad(q, dv), _pad(k, dv), v, 0.9, causal, k_len)
    assert np.array_equal(o, op) and np.array_equal(lse, lp)


def test_value_columns_are_independent():
    """O of V = [V1 | V2] is [O of V1 | O of V2]: the weights do not depend on V."""
    q, k = _rand((1, 2, 6, 4), 7), _rand((1, 2, 10, 4), 8)
    v1, v2 = _rand((1, 2, 10, 2), 9), _rand((1, 2, 10, 5), 10)
    o, lse = oracle.attention_ex(q, k, torch.cat([v1, v2], dim=3).contiguous(), 0.5, True)
    o1, l1 = oracle.attention_ex(q, k, v1, 0.5, True)
    o2, l2 = oracle.attention_ex(q, k, v2, 0.5, True)
    assert np.array_equal(o, np.concatenate([o1, o2], axis=3))
    assert np.array_equal(lse, l1) and np.array_equal(lse, l2)


def _decimal_row(qi, K, V, scale, kept):
    decimal.getcontext().prec = 40
    D = decimal.Decimal
    s = [D(scale) * sum(D(a) * D(b) for a, b in zip(qi, K[j])) for j in kept]
    m = max(s)
    e = [(x - m).exp() for x in s]
    tot = sum(e)
    o = [float(sum(e[t] * D(V[j][c]) for t, j in enumerate(kept)) / tot) for c in range(len(V[0]))]
    return o, float(m + tot.ln())


@pytest.mark.parametrize("dk,dv", [(2, 5), (6, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(dk, dv, causal):
    Nq, Nk, L = 4, 6, 5
    q, k, v = _rand((1, 1, Nq, dk), 11), _rand((1, 1, Nk, dk), 12), _rand((1, 1, Nk, dv), 13)
    o, lse = oracle.attention_ex(q, k, v, 0.7, causal, [L])
    for i in range(Nq):
        kept = [j for j in range(L) if not causal or j <= i + L - Nq]
        ro, rl = _decimal_row(q[0, 0, i].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.7, kept)
        assert np.abs(o[0, 0, i] - ro).max() < 1e-12 and abs(lse[0, 0, i] - rl) < 1e-12


# ------------------------------------------------------------------ gradients
@pytest.mark.parametrize("B,H,Nq,Nk,k_len", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_of_narrow_values_are_the_padded_problem(B, H, Nq, Nk, k_len, causal):
    dk, dv = 6, 2
    q, k = _rand((B, H, Nq, dk), 21), _rand((B, H, Nk, dk), 22)
    v, g = _rand((B, H, Nk, dv), 23), _rand((B, H, Nq, dv), 24)
    dq, dkk, dvv = oracle.attention_bwd_ex(q, k, v, g, 0.8, causal, k_len)
    assert dq.shape == (B, H, Nq, dk) and dkk.shape == (B, H, Nk, dk) and dvv.shape == (B, H, Nk, dv)
    pq, pk, pv = oracle.attention_bwd_ex(q, k, _pad(v, dk), _pad(g, dk), 0.8, causal, k_len)
    assert np.array_equal(dq, pq) and np.array_equal(dkk, pk)
    assert np.array_equal(dvv, pv[..., :dv]) and np.all(pv[..., dv:] == 0)


@pytest.mark.parametrize("B,H,Nq,Nk,k_len", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_of_wide_values_are_the_padded_problem(B, H, Nq, Nk, k_len, causal):
    dk, dv = 2, 7
    q, k = _rand((B, H, Nq, dk), 31), _rand((B, H, Nk, dk), 32)
    v, g = _rand((B, H, Nk, dv), 33), _rand((B, H, Nq, dv), 34)
    dq, dkk, dvv = oracle.attention_bwd_ex(q, k, v, g, 0.8, causal, k_len)
    pq, pk, pv = oracle.attention_bwd_ex(_pad(q, dv), _pad(k, dv), v, g, 0.8, causal, k_len)
    assert np.array_equal(dq, pq[..., :dk]) and np.all(pq[..., dk:] == 0)
    assert np.array_equal(dkk, pk[..., :dk]) and np.all(pk[..., dk:] == 0)
    assert np.array_equal(dvv, pv)


def _loss(q, k, v, g, scale, causal, k_len):
    o, _ = oracle.attention_ex(q, k, v, scale, causal, k_len)
    return float((torch.from_numpy(o) * g).sum())


@pytest.mark.parametrize("dk,dv", [(2, 4), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences_of_the_forward(dk, dv, causal):
    B, H, Nq, Nk, k_len = 2, 1, 4, 5, [5, 3]
    q, k = _rand((B, H, Nq, dk), 41), _rand((B, H, Nk, dk), 42)
    v, g = _rand((B, H, Nk, dv), 43), _rand((B, H, Nq, dv), 44)
    scale = 0.6
    grads = oracle.attention_bwd_ex(q, k, v, g, scale, causal, k_len)
    h = 1e-6
    for name, x, grad in zip("qkv", (q, k, v), grads):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            lp = _loss(*(xp if n == name else args[n] for n in "qkv"), g, scale, causal, k_len)
            lm = _loss(*(xm if n == name else args[n] for n in "qkv"), g, scale, causal, k_len)
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7, (name, np.abs(num - grad).max())


def test_mismatched_value_shapes_are_rejected():
    q, k = _rand((1, 1, 4, 3), 51), _rand((1, 1, 6, 3), 52)
    with pytest.raises(ValueError):  # values of another key count
        oracle.attn_rows_ex(q, k, _rand((1, 1, 5, 2), 53), 1.0, False)
    v = _rand((1, 1, 6, 2), 54)
    with pytest.raises(ValueError):  # dO must have the value head dim
        oracle.attn_bwd_ex(q, k, v, _rand((1, 1, 4, 3), 55), 1.0, False)
