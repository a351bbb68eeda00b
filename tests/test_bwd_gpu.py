"""GPU parity of the gradients: libfa.so's fa_bwd (through its C ABI) against
the fp64 gradient oracle (oracle/oracle_bwd.c).

The oracle differentiates the exact attention of the seeded inputs; the GPU
path differentiates from its own forward outputs (O rounded to the element
type, fp32 lse), as a training step would.  Element-by-element comparisons in
full on small shapes spanning several tiles and ragged tails, and on sampled
rows at the reference workload shapes.
"""
import math

import numpy as np
import pytest
import torch

import exact_attention_29_amd as fa
import oracle
from exact_attention_29_amd.inputs import WORKLOADS, make_dout, make_qkv, workload_inputs
from tests import parity

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def run(q, k, v, g, causal, scale):
    qc, kc, vc, gc = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(qc, kc, vc, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_bwd(qc, kc, vc, o, lse, gc, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def errors(got, ref):
    """|got - ref| statistics relative to the scale of the reference tensor:
    its largest element, or 0.01 if that is smaller (with N(0, 1) inputs a
    gradient tensor is that small only where it vanishes identically, e.g. dq
    and dk at N = 1, and the GPU result is then pure rounding)."""
    g = got.detach().to("cpu").double().numpy().reshape(ref.shape)
    d = np.abs(g - ref)
    big = max(float(np.abs(ref).max()), 1e-2)
    return dict(max_rel=float(d.max()) / big, mean_rel=float(d.mean()) / big, ref_max=big,
                finite=bool(np.isfinite(g).all()))


def check(stats, dtype, name):
    tol = parity.TOL_BWD[dtype]
    print(name, {k: (round(v, 7) if isinstance(v, float) else v) for k, v in stats.items()})
    assert stats["finite"], (name, stats)
    assert stats["max_rel"] <= tol["max_rel"], (name, stats, tol)
    assert stats["mean_rel"] <= tol["mean_rel"], (name, stats, tol)


SMALL = [(dt, d, causal, N) for dt in ("bf16", "fp16") for d in (64, 128) for causal in (False, True)
         for N in (1, 4, 63, 65, 128, 129, 391)]


@pytest.mark.parametrize("dt,d,causal,N", SMALL)
def test_small_shapes_match_gradient_oracle(dt, d, causal, N):
    seed = 2000 + 7 * N + d + int(causal)
    q, k, v = make_qkv(2, 3, N, d, dt, seed)
    g = make_dout(2, 3, N, d, dt, seed + 1)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = run(q, k, v, g, causal, scale)
    rq, rk, rv = oracle.attention_bwd(q, k, v, g, scale, causal)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(errors(got, ref), DT[dt], name)


@pytest.mark.parametrize("dt,B,H,N,d", [("bf16", 2, 4, 333, 128), ("fp32", 1, 1, 1024, 1024)])
def test_gradients_are_bitwise_reproducible(dt, B, H, N, d):
    """No atomics: the same call gives the same bits (the fp32 case runs with
    its query and key tiles split over several workgroups, summed in order)."""
    q, k, v = make_qkv(B, H, N, d, dt, 77)
    g = make_dout(B, H, N, d, dt, 78)
    a = run(q, k, v, g, True, d ** -0.5)
    b = run(q, k, v, g, True, d ** -0.5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_non_default_scale_and_large_scores():
    """scale is applied to the scores only: a scale of 0.3 on N(0,1) inputs of
    d = 64 gives scores of several units and peaked rows."""
    q, k, v = make_qkv(1, 2, 200, 64, "bf16", 91)
    g = make_dout(1, 2, 200, 64, "bf16", 92)
    for causal in (False, True):
        dq, dk, dv = run(q, k, v, g, causal, 0.3)
        rq, rk, rv = oracle.attention_bwd(q, k, v, g, 0.3, causal)
        for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
            check(errors(got, ref), torch.bfloat16, name)


@pytest.mark.parametrize("wl", [3, 4])
def test_workload_shapes_on_sampled_rows(wl):
    """The batched (d = 64) and causal (d = 128, N = 8192) workload shapes,
    launched whole; the oracle computes sampled query rows (dq) and key rows
    (dk, dv) of three heads."""
    w = WORKLOADS[wl]
    q, k, v = workload_inputs(w)
    g = make_dout(w.B, w.H, w.N, w.d, w.dtype, 100 + wl)
    dq, dk, dv = run(q, k, v, g, w.causal, w.scale)
    heads = {(0, 0), (w.B - 1, w.H // 2), (w.B - 1, w.H - 1)}
    rows = parity.sample_rows(w.B, w.H, w.N, seed=wl, per_head_random=48, tile=128,
                              full_tile_heads=heads, heads=heads)
    rq, rk, rv = oracle.attn_bwd(q, k, v, g, w.scale, w.causal, rows, rows)
    flat = lambda t: t.detach().to("cpu").double().reshape(-1, w.d).numpy()[rows]
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(errors(torch.from_numpy(flat(got)), ref), DT[w.dtype], name)


def test_rejected_calls_raise():
    q = torch.zeros(1, 1, 16, 64, device="cuda", dtype=torch.float32)
    o, lse = fa.attention(q, q, q)
    with pytest.raises(ValueError):
        fa.attention_bwd(q, q, q, o, lse, q.to(torch.bfloat16))  # mixed dtypes
    qb = q.to(torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention_bwd(qb, qb, qb, qb, lse[:, :, :8], qb)
    q2 = torch.zeros(1, 1, 16, 2048, device="cuda", dtype=torch.float32)
    with pytest.raises(ValueError):  # no gradient kernel for d = 2048
        fa.attention_bwd(q2, q2, q2, q2, lse, q2)


def check_one_key(dq, dk, q, k, v, g, scale, rq, rk):
    """fp32 problems with one key (Nk = 1): P = 1 on every kept pair and
    dS = dP - delta = 0, so dq and dk vanish identically (the oracle's are
    exact zeros) and the GPU's are fp32 rounding of the two cancelling dot
    products dO.v and dO.o.  Each has error at most gamma_d sum |dO||v|
    (gamma_d ~ d u, the standard bound for a dot product of length d); o = P v
    adds a few ulp of v, and exp2 a few of P: |dS_i| <= (2d + 8) u sum|dO_i| 2|v|
    with u = 2^-24, dq_i = scale dS_i k and dk = scale sum_i dS_i q_i."""
    assert np.abs(rq).max() == 0 and np.abs(rk).max() == 0
    d = q.shape[-1]
    u = 2.0 ** -24
    dS = (2 * d + 8) * u * (g.double().abs() * 2 * v.double().abs()).sum(-1, keepdim=True)
    bq = scale * dS * k.double().abs()
    bk = scale * (dS * q.double().abs()).sum(-2, keepdim=True)
    aq, ak = dq.cpu().double().abs(), dk.cpu().double().abs()
    print("one key: |dq|/bound", float((aq / bq).max()), "|dk|/bound", float((ak / bk).max()))
    assert torch.all(aq <= bq) and torch.all(ak <= bk)


@pytest.mark.parametrize("causal", [False, True])
def test_fp32_d128_large_grid_on_sampled_rows(causal):
    """fp32 at d = 128 with 4096 key blocks of 32: the dK/dV kernel runs its
    one-wave-per-block arrangement there (two waves per block are taken
    only for grids under 4 workgroups per compute unit, 8 when causal; the
    small fp32 shapes below take that one).  The oracle computes sampled
    query rows (dq) and key rows (dk, dv) of three heads."""
    B, H, N, d = 1, 32, 4096, 128
    q, k, v = make_qkv(B, H, N, d, "fp32", 7100 + int(causal))
    g = make_dout(B, H, N, d, "fp32", 7200 + int(causal))
    scale = 1 / math.sqrt(d)
    dq, dk, dv = run(q, k, v, g, causal, scale)
    heads = {(0, 0), (0, H // 2), (0, H - 1)}
    rows = parity.sample_rows(B, H, N, seed=71, per_head_random=32, tile=32,
                              full_tile_heads=heads, heads=heads)
    rq, rk, rv = oracle.attn_bwd(q, k, v, g, scale, causal, rows, rows)
    flat = lambda t: t.detach().to("cpu").double().reshape(-1, d).numpy()[rows]
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(errors(torch.from_numpy(flat(got)), ref), torch.float32, name)


# ------------------------------------------------------------------ fp32
# fp32 inputs run every product in full fp32 (v_mfma_f32_32x32x2_f32): the
# only error sources are fp32 rounding of the sums and of exp2, so the
# gradients are held to 1e-4 of their scale (as the fp32 forward output is
# held to 1e-4), with a mean bound ten times tighter.
FP32 = [(d, causal, N) for d in (64, 128, 256, 512, 1024) for causal in (False, True)
        for N in (1, 65, 200)]


@pytest.mark.parametrize("d,causal,N", FP32)
def test_fp32_shapes_match_gradient_oracle(d, causal, N):
    seed = 6000 + 7 * N + d + int(causal)
    B, H = (2, 3) if d <= 256 else (1, 2)
    q, k, v = make_qkv(B, H, N, d, "fp32", seed)
    g = make_dout(B, H, N, d, "fp32", seed + 1)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = run(q, k, v, g, causal, scale)
    rq, rk, rv = oracle.attention_bwd(q, k, v, g, scale, causal)
    if N == 1:
        check_one_key(dq, dk, q, k, v, g, scale, rq, rk)
        check(errors(dv, rv), torch.float32, "dv")
        return
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(errors(got, ref), torch.float32, name)


# ------------------------------------------------------------------ unequal lengths, key padding
@pytest.mark.parametrize("dt,d", [("bf16", 64), ("bf16", 128), ("fp16", 128), ("fp32", 64),
                                  ("fp32", 512)])
@pytest.mark.parametrize("Nq,Nk,k_len", [(77, 300, None), (300, 77, None), (129, 1, None),
                                         (190, 333, [333, 150, 0]), (64, 64, [40, 64, 1])])
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_lengths_and_padding_match_gradient_oracle(dt, d, Nq, Nk, k_len, causal):
    B, H = 3, 2
    seed = 5000 + Nq + 3 * Nk + d + int(causal)
    q, _, _ = make_qkv(B, H, Nq, d, dt, seed)
    _, k, v = make_qkv(B, H, Nk, d, dt, seed + 1)
    g = make_dout(B, H, Nq, d, dt, seed + 2)
    scale = 1 / math.sqrt(d)
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device="cuda")
    qc, kc, vc, gc = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(qc, kc, vc, causal=causal, scale=scale, k_len=kl)
    dq, dk, dv = fa.attention_bwd(qc, kc, vc, o, lse, gc, causal=causal, scale=scale, k_len=kl)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_bwd_ex(q, k, v, g, scale, causal, k_len)
    vanish = dt == "fp32" and Nk == 1  # see check_one_key
    if vanish:
        check_one_key(dq, dk, q, k, v, g, scale, rq, rk)
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        if not (vanish and name != "dv"):
            check(errors(got, ref), DT[dt], name)
    # structural zeros are exact: keys past a batch's count (no query keeps
    # them) and query rows that keep no key
    lens = [Nk] * B if k_len is None else [min(max(x, 0), Nk) for x in k_len]
    for b, L in enumerate(lens):
        assert torch.all(dk[b, :, L:] == 0) and torch.all(dv[b, :, L:] == 0)
        empty = [i for i in range(Nq) if L == 0 or (causal and i + L - Nq < 0)]
        assert torch.all(dq[b, :, empty] == 0)


# ------------------------------------------------------------------ value head dim of its own
def dv_inputs(B, H, Nq, Nk, dk, dv, dt, seed):
    q, k, _ = make_qkv(B, H, max(Nq, Nk), dk, dt, seed)
    _, _, v = make_qkv(B, H, Nk, dv, dt, seed + 1)
    g = make_dout(B, H, Nq, dv, dt, seed + 2)
    return q[:, :, :Nq].contiguous(), k[:, :, :Nk].contiguous(), v, g


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
@pytest.mark.parametrize("Nq,Nk,k_len", [(200, 200, None), (77, 300, None), (300, 77, None),
                                         (190, 333, [333, 150, 0])])
@pytest.mark.parametrize("causal", [False, True])
def test_unequal_head_dims_match_gradient_oracle(dt, dk, dv, Nq, Nk, k_len, causal):
    B, H = 3, 2
    q, k, v, g = dv_inputs(B, H, Nq, Nk, dk, dv, dt, 8000 + Nq + 3 * Nk + dk + int(causal))
    scale = 1 / math.sqrt(dk)
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device="cuda")
    qc, kc, vc, gc = (t.cuda() for t in (q, k, v, g))
    o, lse = fa.attention(qc, kc, vc, causal=causal, scale=scale, k_len=kl)
    dq, dk_, dv_ = fa.attention_bwd(qc, kc, vc, o, lse, gc, causal=causal, scale=scale, k_len=kl)
    torch.cuda.synchronize()
    assert dq.shape == q.shape and dk_.shape == k.shape and dv_.shape == v.shape
    rq, rk, rv = oracle.attention_bwd_ex(q, k, v, g, scale, causal, k_len)
    for name, got, ref in (("dq", dq, rq), ("dk", dk_, rk), ("dv", dv_, rv)):
        check(errors(got, ref), DT[dt], name)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_narrow_qk_gradients_equal_the_zero_padded_equal_dim_call(dt, causal):
    """d_qk = 64, d_v = 128 against d = 128 with Q and K zero beyond column 64
    (same o, lse, dO): the extra score columns add exact zeros, so dq and dk
    are the first 64 columns of the padded call's, the rest zero, and dv is
    equal, all bit for bit in bf16.  In fp32 the padded call's kernels split
    the 128 columns over two waves and add their partial dP in LDS, where the
    narrow call accumulates dP in one chain, so dq and dk agree to rounding
    (dv, computed column by column from the same P, stays bitwise equal)."""
    B, H, N = 2, 4, 700
    q, k, v, g = (t.cuda() for t in dv_inputs(B, H, N, N, 64, 128, dt, 8100 + int(causal)))
    o, lse = fa.attention(q, k, v, causal=causal, scale=0.1)
    a = fa.attention_bwd(q, k, v, o, lse, g, causal=causal, scale=0.1)
    pad = lambda x: torch.cat([x, torch.zeros_like(x)], dim=3).contiguous()
    b = fa.attention_bwd(pad(q), pad(k), v, o, lse, g, causal=causal, scale=0.1)
    torch.cuda.synchronize()
    for i in (0, 1):
        assert torch.all(b[i][..., 64:] == 0)
        if dt == "bf16":
            assert torch.equal(a[i], b[i][..., :64])
        else:  # two fp32 sums of the same terms in different orders
            scale_i = b[i].abs().max().item()
            assert (a[i] - b[i][..., :64]).abs().max().item() <= 1e-6 * scale_i
    assert torch.equal(a[2], b[2])


def test_small_grids_take_the_split_and_match_the_oracle():
    """Few heads and long rows: fewer key (query) blocks than the GPU holds,
    so each block's tiles are shared out and the fp32 partial sums added; the
    workspace then holds more than the two row statistics."""
    B, H, N, d = 1, 2, 1500, 128
    stats = 2 * B * H * ((N + 31) // 32 * 32) * 4
    assert fa.fa_bwd_workspace_size(B, H, N, d, 1, fa.FA_DTYPE_BF16) > stats
    q, k, v = make_qkv(B, H, N, d, "bf16", 4321)
    g = make_dout(B, H, N, d, "bf16", 4322)
    dq, dk, dv = run(q, k, v, g, True, d ** -0.5)
    rows = parity.sample_rows(B, H, N, seed=5, per_head_random=40, tile=128)
    rq, rk, rv = oracle.attn_bwd(q, k, v, g, d ** -0.5, True, rows, rows)
    flat = lambda t: t.detach().to("cpu").double().reshape(-1, d).numpy()[rows]
    for name, got, ref in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        check(errors(torch.from_numpy(flat(got)), ref), torch.bfloat16, name)
