"""Pins of the fp64 gradient oracle (oracle/oracle_bwd.c), CPU only.

The gradient oracle is checked against things other than its own formula:
central finite differences of the forward oracle (the definition of a
derivative, independent of the chain rule written in oracle_bwd.c), a
library's automatic differentiation of the materialised attention, closed
forms, and an invariance of the softmax.
"""
import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


def _loss(q, k, v, g, scale, causal):
    """L = sum(dL/dO * O) with O from the forward oracle."""
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float((torch.from_numpy(o) * g).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_central_differences_of_the_forward(causal):
    B, H, N, d = 1, 2, 5, 3
    q, k, v, g = (_rand((B, H, N, d), s) for s in (1, 2, 3, 4))
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(grad)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.clone(), x.clone()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, scale, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], g, scale, causal)) / (2 * h)
        assert np.abs(num - grad).max() < 1e-7, (name, np.abs(num - grad).max())


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_autograd_of_the_materialised_attention(causal):
    B, H, N, d = 1, 2, 40, 8
    q, k, v, g = (_rand((B, H, N, d), s) for s in (11, 12, 13, 14))
    scale = d ** -0.5
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    s = scale * qa @ ka.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ va
    o.backward(g)
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, scale, causal)
    for ref, got in ((qa.grad, dq), (ka.grad, dk), (va.grad, dv)):
        assert np.abs(ref.numpy() - got).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_key_gradients_sum_to_zero(causal):
    """Adding one vector to every key shifts each row's kept scores by a
    constant, which the softmax ignores: the key gradients sum to zero."""
    B, H, N, d = 2, 2, 17, 5
    q, k, v, g = (_rand((B, H, N, d), s) for s in (21, 22, 23, 24))
    _, dk, _ = oracle.attention_bwd(q, k, v, g, 0.4, causal)
    assert np.abs(dk.sum(axis=2)).max() < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_averaging_closed_forms(causal):
    """Q = 0: every kept weight of row i is 1/|J_i|, so dV_j is the sum of
    dO_i/|J_i| over the rows that keep key j, and dK = scale*dS^T Q = 0."""
    B, H, N, d = 1, 1, 9, 4
    k, v, g = (_rand((B, H, N, d), s) for s in (31, 32, 33))
    q = torch.zeros_like(k)
    _, dk, dv = oracle.attention_bwd(q, k, v, g, 0.5, causal)
    gg = g[0, 0].numpy()
    for j in range(N):
        rows = range(j, N) if causal else range(N)
        expect = sum(gg[i] / ((i + 1) if causal else N) for i in rows)
        assert np.abs(dv[0, 0, j] - expect).max() < 1e-13
    assert np.abs(dk).max() < 1e-13


def test_row_subsets_and_linearity_in_the_upstream_gradient():
    B, H, N, d = 2, 3, 23, 6
    q, k, v, g = (_rand((B, H, N, d), s) for s in (41, 42, 43, 44))
    dq, dk, dv = oracle.attention_bwd(q, k, v, g, 0.3, True)
    rows = np.array([5, 40, 69, 100, 137], dtype=np.int64)
    sq, sk, sv = oracle.attn_bwd(q, k, v, g, 0.3, True, q_rows=rows, k_rows=rows[::-1].copy())
    flat = lambda a: a.reshape(-1, d)
    assert np.array_equal(sq, flat(dq)[rows])
    assert np.array_equal(sk, flat(dk)[rows[::-1]]) and np.array_equal(sv, flat(dv)[rows[::-1]])
    dq2, dk2, dv2 = oracle.attention_bwd(q, k, v, 2 * g, 0.3, True)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.abs(2 * a - b).max() < 1e-12


def test_low_precision_inputs_are_widened_exactly():
    B, H, N, d = 1, 1, 12, 8
    q, k, v, g = (_rand((B, H, N, d), s, torch.bfloat16) for s in (51, 52, 53, 54))
    a = oracle.attention_bwd(q, k, v, g, 0.35, False)
    b = oracle.attention_bwd(*(t.double() for t in (q, k, v, g)), 0.35, False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_invalid_arguments_are_rejected():
    q = _rand((1, 1, 4, 2), 61)
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, q, q, q, 1.0, False, q_rows=[4])
    with pytest.raises(ValueError):
        oracle.attn_bwd(q, q, q, q[..., :1].contiguous(), 1.0, False)
