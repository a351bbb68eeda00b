"""fp64 tiled online-softmax recurrence -- a test helper, independent of both
the oracle (which runs three passes) and the GPU kernels.

Written from the tiled loop of "The Details of Flash Attention" (section
"Tiling the Loop": running max, running denominator rescaled by
exp(m_old - m_new), tile sums of exp(x - m_new)) and from the worked example of
"Deep Learning - Flash Attention" (section "An Example", steps 4-6: the
unnormalized accumulator O <- alpha*O + P V_j, l <- alpha*l + rowsum(P), and a
final divide by l).  Two loop orders are offered: query-block outer (one worker
per query block, "An Example" step 7) and key/value-block outer (the order of
the numpy listing in "FlashAttention" (ai360xpert), section "Show Me the
Code").  A normalized-accumulator variant follows the output recurrence of
"The Details of Flash Attention", section "Fusing the Output Accumulator".

Every intermediate can be recorded, so tests can compare the per-step maxima
and rescale factors against the numbers printed in the worked example.
"""
from __future__ import annotations

import numpy as np


def _mask(s, q0, k0, causal, n_keys):
    """-inf where key > query (causal) or key index is past the sequence."""
    if not causal:
        return s
    rows = np.arange(q0, q0 + s.shape[0])[:, None]
    cols = np.arange(k0, k0 + s.shape[1])[None, :]
    return np.where(cols <= rows, s, -np.inf)


def _safe_offset(m_new):
    # A row whose every score so far was masked keeps m = -inf; use 0 as its
    # exponent offset so that exp(-inf - 0) = 0 and no -inf - (-inf) occurs.
    return np.where(np.isneginf(m_new), 0.0, m_new)


def tiled_q_outer(q, k, v, scale, causal=False, br=2, bc=2, trace=None):
    """q, k, v: [N, d] float64.  Returns (O, lse)."""
    N = q.shape[0]
    O = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for q0 in range(0, N, br):
        qi = q[q0:q0 + br]
        m = np.full(qi.shape[0], -np.inf)
        l = np.zeros(qi.shape[0])
        acc = np.zeros((qi.shape[0], v.shape[1]))
        for k0 in range(0, N, bc):
            s = _mask(qi @ k[k0:k0 + bc].T * scale, q0, k0, causal, N)
            m_new = np.maximum(m, s.max(axis=1))
            off = _safe_offset(m_new)
            p = np.exp(s - off[:, None])
            alpha = np.exp(m - off)
            l = alpha * l + p.sum(axis=1)
            acc = alpha[:, None] * acc + p @ v[k0:k0 + bc]
            if trace is not None:
                trace.append({"q0": q0, "k0": k0, "s": s.copy(), "m_new": m_new.copy(),
                              "alpha": alpha.copy(), "p": p.copy(), "l": l.copy()})
            m = m_new
        O[q0:q0 + br] = acc / l[:, None]
        lse[q0:q0 + br] = m + np.log(l)
    return O, lse


def tiled_kv_outer(q, k, v, scale, causal=False, br=2, bc=2):
    """Same result with the key/value blocks as the outer loop; the per-row
    state (m, l, O) persists across the outer loop."""
    N = q.shape[0]
    O = np.zeros((N, v.shape[1]))
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    for k0 in range(0, N, bc):
        kj, vj = k[k0:k0 + bc], v[k0:k0 + bc]
        for q0 in range(0, N, br):
            sl = slice(q0, q0 + br)
            s = _mask(q[sl] @ kj.T * scale, q0, k0, causal, N)
            m_new = np.maximum(m[sl], s.max(axis=1))
            off = _safe_offset(m_new)
            p = np.exp(s - off[:, None])
            alpha = np.exp(m[sl] - off)
            O[sl] = alpha[:, None] * O[sl] + p @ vj
            l[sl] = alpha * l[sl] + p.sum(axis=1)
            m[sl] = m_new
    return O / l[:, None], m + np.log(l)


def tiled_normalized(q, k, v, scale, causal=False, bc=2):
    """Row-by-row normalized accumulator: o' <- o' * (d'_old e^{m_old-m_new} / d'_new)
    + sum_j e^{x_j - m_new} / d'_new * V_j, one key block of width bc at a time."""
    N = q.shape[0]
    O = np.zeros((N, v.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        m, dd = -np.inf, 0.0
        o = np.zeros(v.shape[1])
        for k0 in range(0, N, bc):
            x = k[k0:k0 + bc] @ q[i] * scale
            if causal:
                x = np.where(np.arange(k0, k0 + x.shape[0]) <= i, x, -np.inf)
            m_new = max(m, x.max())
            off = 0.0 if np.isneginf(m_new) else m_new
            e = np.exp(x - off)
            d_new = dd * np.exp(m - off) + e.sum()
            if d_new > 0:
                o = o * (dd * np.exp(m - off) / d_new) + (e / d_new) @ v[k0:k0 + bc]
            m, dd = m_new, d_new
        O[i] = o
        lse[i] = m + np.log(dd)
    return O, lse
