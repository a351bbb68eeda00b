"""Pins of the gradient oracle's unequal-length and key-padding extension
(oracle_attn_bwd_ex), CPU only: central finite differences of the extended
forward oracle (the definition of the derivative, independent of the chain
rule the gradient oracle writes out), the plain gradient oracle on derived
problems, and the softmax's shift invariance."""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _loss(q, k, v, g, scale, causal, k_len):
    o, _ = oracle.attention_ex(q, k, v, scale, causal, k_len)
    return float((torch.from_numpy(o) * g).sum())


@pytest.mark.parametrize("Nq,Nk,k_len", [(3, 6, None), (6, 3, None), (4, 7, [5, 0]), (5, 5, [2, 5])])
@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences_of_the_forward(Nq, Nk, k_len, causal):
    B, H, d = 2, 1, 3
    q, g = _rand((B, H, Nq, d), 1), _rand((B, H, Nq, d), 4)
    k, v = _rand((B, H, Nk, d), 2), _rand((B, H, Nk, d), 3)
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd_ex(q, k, v, g, scale, causal, k_len)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            lp = _loss(*(xp if n == name else args[n] for n in "qkv"), g, scale, causal, k_len)
            lm = _loss(*(xm if n == name else args[n] for n in "qkv"), g, scale, causal, k_len)
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7, (name, np.abs(num - grad).max())


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_without_padding_is_the_plain_gradient_oracle(causal):
    q, k, v, g = (_rand((1, 2, 21, 5), s) for s in (11, 12, 13, 14))
    a = oracle.attention_bwd(q, k, v, g, 0.4, causal)
    b = oracle.attention_bwd_ex(q, k, v, g, 0.4, causal)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("causal", [False, True])
def test_padding_equals_truncated_keys_and_padded_keys_get_no_gradient(causal):
    B, H, Nq, Nk, d = 3, 2, 9, 16, 4
    q, g = _rand((B, H, Nq, d), 21), _rand((B, H, Nq, d), 24)
    k, v = _rand((B, H, Nk, d), 22), _rand((B, H, Nk, d), 23)
    k_len = [16, 6, 0]
    dq, dk, dv = oracle.attention_bwd_ex(q, k, v, g, 0.5, causal, k_len)
    for b, L in enumerate(k_len):
        assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)
        if L == 0:
            assert np.all(dq[b] == 0)
            continue
        tq, tk, tv = oracle.attention_bwd_ex(q[b:b + 1], k[b:b + 1, :, :L].contiguous(),
                                             v[b:b + 1, :, :L].contiguous(), g[b:b + 1], 0.5, causal)
        assert np.array_equal(dq[b:b + 1], tq)
        assert np.array_equal(dk[b:b + 1, :, :L], tk) and np.array_equal(dv[b:b + 1, :, :L], tv)


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero_with_unequal_lengths(causal):
    """Adding one vector to every key shifts each row's kept scores by a
    constant: the key gradients of each head sum to zero."""
    q, g = _rand((2, 2, 7, 4), 31), _rand((2, 2, 7, 4), 34)
    k, v = _rand((2, 2, 12, 4), 32), _rand((2, 2, 12, 4), 33)
    _, dk, _ = oracle.attention_bwd_ex(q, k, v, g, 0.6, causal, [12, 5])
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
