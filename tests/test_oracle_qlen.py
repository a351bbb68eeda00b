"""Pins of the oracle's per-batch query counts (q_len of oracle_attn_rows_gen
and oracle_attn_bwd_gen), CPU only.

The mask of the ScaledDotProductAttention listing in "Transformer Attention: A
Mathematical Deep Dive" covers padding; a padded batch holds Lq <= Nq real
queries and L <= Nk real keys.  The reading: a query row at or past Lq is
padding and keeps no key (o = 0, lse = -inf, dq = 0, and it adds nothing to
dk, dv), and the causal diagonal aligns the last real query with the last real
key.  Each batch of such a problem is therefore, bit for bit, the unpadded
problem of its own Lq queries and L keys -- a problem the plain oracles
(pinned elsewhere against closed forms and brute force) compute.  Beside that
reduction: a decimal brute force whose kept set is written out here, and
central differences of the forward for the gradients.
"""
import decimal

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


CASES = [  # B, H, Nq, Nk, q_len, k_len
    (3, 2, 9, 9, [9, 4, 0], None),
    (3, 1, 7, 12, [7, 3, 5], [12, 5, 2]),
    (2, 2, 11, 6, [2, 11], [6, 1]),
    (2, 1, 5, 5, [1, 5], [0, 5]),
]


@pytest.mark.parametrize("B,H,Nq,Nk,q_len,k_len", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_each_batch_is_the_unpadded_problem_of_its_own_lengths(B, H, Nq, Nk, q_len, k_len, causal):
    dk, dv = 5, 3
    q, k, v = _rand((B, H, Nq, dk), 1), _rand((B, H, Nk, dk), 2), _rand((B, H, Nk, dv), 3)
    o, lse = oracle.attention_ex(q, k, v, 0.7, causal, k_len, q_len=q_len)
    for b in range(B):
        Lq, L = q_len[b], Nk if k_len is None else k_len[b]
        pad_o, pad_l = o[b, :, Lq:], lse[b, :, Lq:]
        assert np.all(pad_o == 0) and np.all(np.isneginf(pad_l)), "padding rows"
        if Lq == 0:
            continue
        if L == 0:
            assert np.all(o[b, :, :Lq] == 0) and np.all(np.isneginf(lse[b, :, :Lq]))
            continue
        ot, lt = oracle.attention_ex(q[b:b + 1, :, :Lq].contiguous(), k[b:b + 1, :, :L].contiguous(),
                                     v[b:b + 1, :, :L].contiguous(), 0.7, causal)
        assert np.array_equal(o[b, :, :Lq], ot[0]) and np.array_equal(lse[b, :, :Lq], lt[0])


@pytest.mark.parametrize("causal", [False, True])
def test_full_counts_are_no_counts(causal):
    q, k, v = _rand((2, 2, 6, 4), 4), _rand((2, 2, 8, 4), 5), _rand((2, 2, 8, 4), 6)
    a = oracle.attention_ex(q, k, v, 0.5, causal, [8, 3])
    b = oracle.attention_ex(q, k, v, 0.5, causal, [8, 3], q_len=[6, 6])
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = oracle.attention_ex(q, k, v, 0.5, causal, [8, 3], q_len=[60, 6])  # clamped to Nq
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def _decimal_row(qi, K, V, scale, kept):
    decimal.getcontext().prec = 40
    D = decimal.Decimal
    s = [D(scale) * sum(D(a) * D(b) for a, b in zip(qi, K[j])) for j in kept]
    m = max(s)
    e = [(x - m).exp() for x in s]
    tot = sum(e)
    o = [float(sum(e[t] * D(V[j][c]) for t, j in enumerate(kept)) / tot) for c in range(len(V[0]))]
    return o, float(m + tot.ln())


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    Nq, Nk, Lq, L = 6, 7, 4, 5
    q, k, v = _rand((1, 1, Nq, 3), 7), _rand((1, 1, Nk, 3), 8), _rand((1, 1, Nk, 2), 9)
    o, lse = oracle.attention_ex(q, k, v, 0.8, causal, [L], q_len=[Lq])
    for i in range(Nq):
        # query i < Lq keeps key j < L, and j <= i + (L - Lq) when causal
        kept = [j for j in range(L) if i < Lq and (not causal or j - i <= L - Lq)]
        if not kept:
            assert np.all(o[0, 0, i] == 0) and np.isneginf(lse[0, 0, i])
            continue
        ro, rl = _decimal_row(q[0, 0, i].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), 0.8, kept)
        assert np.abs(o[0, 0, i] - ro).max() < 1e-12 and abs(lse[0, 0, i] - rl) < 1e-12


# ------------------------------------------------------------------ gradients
@pytest.mark.parametrize("B,H,Nq,Nk,q_len,k_len", CASES)
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_of_each_batch_are_the_unpadded_problem(B, H, Nq, Nk, q_len, k_len, causal):
    dk, dv = 4, 6
    q, k = _rand((B, H, Nq, dk), 11), _rand((B, H, Nk, dk), 12)
    v, g = _rand((B, H, Nk, dv), 13), _rand((B, H, Nq, dv), 14)
    dq, dkk, dvv = oracle.attention_bwd_ex(q, k, v, g, 0.6, causal, k_len, q_len=q_len)
    for b in range(B):
        Lq, L = q_len[b], Nk if k_len is None else k_len[b]
        assert np.all(dq[b, :, Lq:] == 0), "padding rows have no gradient"
        assert np.all(dkk[b, :, L:] == 0) and np.all(dvv[b, :, L:] == 0), "padding keys"
        if Lq == 0 or L == 0:
            assert np.all(dq[b] == 0) and np.all(dkk[b] == 0) and np.all(dvv[b] == 0)
            continue
        tq, tk, tv = oracle.attention_bwd_ex(
            q[b:b + 1, :, :Lq].contiguous(), k[b:b + 1, :, :L].contiguous(),
            v[b:b + 1, :, :L].contiguous(), g[b:b + 1, :, :Lq].contiguous(), 0.6, causal)
        assert np.array_equal(dq[b, :, :Lq], tq[0])
        assert np.array_equal(dkk[b, :, :L], tk[0]) and np.array_equal(dvv[b, :, :L], tv[0])


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences_of_the_forward(causal):
    B, H, Nq, Nk, q_len, k_len = 2, 1, 5, 4, [3, 5], [4, 2]
    q, k = _rand((B, H, Nq, 2), 21), _rand((B, H, Nk, 2), 22)
    v, g = _rand((B, H, Nk, 3), 23), _rand((B, H, Nq, 3), 24)
    scale = 0.9

    def loss(qq, kk, vv):
        o, _ = oracle.attention_ex(qq, kk, vv, scale, causal, k_len, q_len=q_len)
        return float((torch.from_numpy(o) * g).sum())

    grads = oracle.attention_bwd_ex(q, k, v, g, scale, causal, k_len, q_len=q_len)
    h = 1e-6
    for n, grad in enumerate(grads):
        x = (q, k, v)[n]
        num = np.zeros_like(grad)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[n], args_m[n] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7, ("qkv"[n], np.abs(num - grad).max())


def test_count_shapes_are_checked():
    q = _rand((2, 1, 4, 3), 31)
    with pytest.raises(ValueError):
        oracle.attn_rows_ex(q, q, q, 1.0, False, q_len=[4])
    with pytest.raises(ValueError):
        oracle.attn_bwd_ex(q, q, q, q, 1.0, False, q_len=[1, 2, 3])
