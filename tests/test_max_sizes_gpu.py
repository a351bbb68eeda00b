"""GPU parity at the largest sizes the boundary accepts: a key sequence whose
per-head byte offsets reach the 32-bit offsets of the buffer loads
((Nk + 128) * d * element size just below 2^31), with two heads so that the
second head's rows start past 2^31 bytes, for the forward and the gradients.

A few query blocks against ~8.4 million keys (bf16, d = 128) or ~4.2 million
(fp32): the oracle computes sampled rows in full (about 2 GFLOP of fp64 per
query row).  The first key past the limit is rejected on the host.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_29_amd as fa
import oracle
from exact_attention_29_amd.inputs import make_normal_device
from tests import parity

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def max_keys(d, elem):
    """Largest Nk with (Nk + 128) * d * elem <= 2^31 - 1."""
    return (0x7fffffff // (d * elem)) - 128


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_forward_at_the_largest_key_count(dt, causal):
    d, elem = 128, (2 if dt == "bf16" else 4)
    B, H, Nq, Nk = 1, 2, 200, max_keys(d, elem)
    print(f"forward {dt} causal={causal} Nq={Nq} Nk={Nk}", flush=True)
    q = make_normal_device((B, H, Nq, d), dt, 11)
    k = make_normal_device((B, H, Nk, d), dt, 12)
    v = make_normal_device((B, H, Nk, d), dt, 13)
    scale = 1 / math.sqrt(d)
    o, lse = fa.attention(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    rows = np.array([0, 1, 63, 64, 127, 128, 199, Nq + 0, Nq + 77, 2 * Nq - 1], dtype=np.int64)
    o_ref, l_ref = oracle.attn_rows_ex(qh, kh, vh, scale, causal, rows)
    og = o.double().cpu().reshape(-1, d).numpy()[rows]
    lg = lse.double().cpu().reshape(-1).numpy()[rows]
    do = np.abs(og - o_ref)
    parity.check(dict(max_o=float(do.max()), mean_o=float(do.mean()),
                      max_lse=float(np.abs(lg - l_ref).max()), finite=bool(np.isfinite(og).all()),
                      rows=len(rows)), DT[dt])


def test_gradients_at_the_largest_key_count():
    d, dt = 128, "bf16"
    B, H, Nq, Nk = 1, 2, 32, max_keys(d, 2)
    print(f"gradients {dt} Nq={Nq} Nk={Nk}", flush=True)
    q = make_normal_device((B, H, Nq, d), dt, 21)
    k = make_normal_device((B, H, Nk, d), dt, 22)
    v = make_normal_device((B, H, Nk, d), dt, 23)
    g = make_normal_device((B, H, Nq, d), dt, 24)
    scale = 1 / math.sqrt(d)
    o, lse = fa.attention(q, k, v, causal=True, scale=scale)
    dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, g, causal=True, scale=scale)
    torch.cuda.synchronize()
    qh, kh, vh, gh = q.cpu(), k.cpu(), v.cpu(), g.cpu()
    q_rows = np.array([0, 31, Nq + 5, 2 * Nq - 1], dtype=np.int64)
    # keys at both ends of each head, including the last rows past 2^31 bytes
    k_rows = np.array([0, 1, Nk - 40, Nk - 1, Nk, Nk + 12345, 2 * Nk - 2, 2 * Nk - 1],
                      dtype=np.int64)
    rq, rk, rv = oracle.attn_bwd_ex(qh, kh, vh, gh, scale, True, q_rows, k_rows)
    flat = lambda t: t.detach().cpu().double().reshape(-1, d).numpy()
    for name, got, ref in (("dq", flat(dq)[q_rows], rq), ("dk", flat(dk)[k_rows], rk),
                           ("dv", flat(dv)[k_rows], rv)):
        big = max(float(np.abs(ref).max()), 1e-2)
        err = np.abs(got - ref)
        stats = dict(max_rel=float(err.max()) / big, mean_rel=float(err.mean()) / big)
        print(name, stats)
        assert np.isfinite(got).all()
        assert stats["max_rel"] <= parity.TOL_BWD[torch.bfloat16]["max_rel"], (name, stats)
