"""GPU test of the allocation-free forward entry point, fa_fwd_gen_noalloc,
through the C ABI: its outputs equal fa_fwd_gen's (with a workspace of
fa_fwd_gen_workspace_size bytes) bit for bit, on two split calls in a row --
the second smaller than the first, so it runs on what the first left in the
library's scratch -- and agree with the fp64 oracle within the workload
tolerance.  A problem whose split would need more than the scratch holds is
rejected before any launch.
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
CODE = {"bf16": fa.FA_DTYPE_BF16, "fp16": fa.FA_DTYPE_FP16, "fp32": fa.FA_DTYPE_FP32}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def ptr(t):
    return None if t is None else t.data_ptr()


def run_pair(B, H, Nq, Nk, dk, dv, dt, causal, k_len=None, q_len=None, seed=0):
    """(noalloc outputs, fa_fwd_gen outputs, host inputs, scale) of one problem."""
    q, k, _ = make_qkv(B, H, max(Nq, Nk), dk, dt, seed)
    _, _, v = make_qkv(B, H, Nk, dv, dt, seed + 1)
    q, k = q[:, :, :Nq].contiguous(), k[:, :, :Nk].contiguous()
    dev = torch.device("cuda")
    qc, kc, vc = q.to(dev), k.to(dev), v.to(dev)
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device=dev)
    ql = None if q_len is None else torch.tensor(q_len, dtype=torch.int32, device=dev)
    scale = 1 / math.sqrt(dk)
    stream = torch.cuda.current_stream().cuda_stream
    code, c = CODE[dt], int(causal)
    ws_bytes = fa.fa_fwd_gen_workspace_size(B, H, Nq, Nk, dk, dv, c, code)
    assert 0 < ws_bytes <= fa.FA_NOALLOC_SCRATCH_BYTES, ws_bytes  # a split that fits
    o1 = torch.full((B, H, Nq, dv), float("nan"), dtype=DT[dt], device=dev)
    l1 = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    st = fa.fa_fwd_gen_noalloc(ptr(qc), ptr(kc), ptr(vc), ptr(o1), ptr(l1), B, H, Nq, Nk, dk, dv,
                               scale, c, code, ptr(kl), ptr(ql), stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = fa.fa_fwd_gen(ptr(qc), ptr(kc), ptr(vc), ptr(o2), ptr(l2), B, H, Nq, Nk, dk, dv, scale,
                       c, code, ptr(kl), ptr(ql), ptr(ws), ws_bytes, stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2), (q, k, v), scale


def check_oracle(o, lse, q, k, v, scale, causal, dt, k_len=None, q_len=None, rows=None):
    o_ref, l_ref = oracle.attn_rows_ex(q, k, v, scale, causal, rows, k_len, q_len=q_len)
    dv = v.shape[-1]
    og = o.double().cpu().reshape(-1, dv).numpy()
    lg = lse.double().cpu().reshape(-1).numpy()
    if rows is not None:
        og, lg = og[rows], lg[rows]
    empty = np.isneginf(l_ref)
    assert np.all(og[empty] == 0) and np.all(np.isneginf(lg[empty]))
    do = np.abs(og[~empty] - o_ref[~empty])
    dl = np.abs(lg[~empty] - l_ref[~empty])
    st = dict(max_o=float(do.max()), mean_o=float(do.mean()), max_lse=float(dl.max()),
              rows=int(o_ref.shape[0]), finite=bool(np.isfinite(og).all()))
    print(st)
    parity.check(st, DT[dt])


def test_noalloc_equals_workspace_call_twice():
    # first call: a split of a causal bf16 d = 128 problem (4 heads of 8192
    # rows: fewer 256-row blocks than compute units)
    print("noalloc call 1: bf16 B1 H4 N8192 d128 causal", flush=True)
    (o1, l1), (o2, l2), (q, k, v), scale = run_pair(1, 4, 8192, 8192, 128, 128, "bf16", True,
                                                    seed=41)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rows = parity.sample_rows(1, 4, 8192, seed=3, per_head_random=48, tile=256)
    check_oracle(o1, l1, q, k, v, scale, True, "bf16", rows=rows)
    # second call, smaller, on the scratch the first call left behind:
    # fp32, the one-head 128-row shape, keys split in one-tile ranges
    print("noalloc call 2: fp32 B1 H1 N128 d64", flush=True)
    (o1, l1), (o2, l2), (q, k, v), scale = run_pair(1, 1, 128, 128, 64, 64, "fp32", False,
                                                    seed=43)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check_oracle(o1, l1, q, k, v, scale, False, "fp32")


def test_noalloc_counts_and_head_dims():
    # 16-bit split with per-batch key and query counts and d_qk != d_v
    print("noalloc: bf16 B2 H2 Nq700 Nk3000 d64/128 causal, counts", flush=True)
    k_len, q_len = [3000, 1700], [700, 333]
    (o1, l1), (o2, l2), (q, k, v), scale = run_pair(2, 2, 700, 3000, 64, 128, "bf16", True,
                                                    k_len=k_len, q_len=q_len, seed=45)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    check_oracle(o1, l1, q, k, v, scale, True, "bf16", k_len=k_len, q_len=q_len)


def test_noalloc_unsplit_grid_and_oversized_split():
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # a grid that fills the device runs unsplit (no scratch) and equals fa_fwd
    print("noalloc: unsplit bf16 B2 H16 N4096 d128", flush=True)
    q, k, v = (t.to(dev) for t in make_qkv(2, 16, 4096, 128, "bf16", 47))
    assert fa.fa_fwd_gen_workspace_size(2, 16, 4096, 4096, 128, 128, 1, fa.FA_DTYPE_BF16) == 0
    o1, l1 = torch.empty_like(q), torch.empty((2, 16, 4096), device=dev)
    st = fa.fa_fwd_gen_noalloc(ptr(q), ptr(k), ptr(v), ptr(o1), ptr(l1), 2, 16, 4096, 4096, 128,
                               128, 1 / math.sqrt(128), 1, fa.FA_DTYPE_BF16, None, None, stream)
    assert st == fa.FA_OK
    o2, l2 = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # a split larger than the scratch is refused before any launch
    B, H, N = 1, 85, 768  # 255 blocks of 256 rows, two shares: 67.4 MB
    need = fa.fa_fwd_gen_workspace_size(B, H, N, N, 128, 128, 0, fa.FA_DTYPE_BF16)
    print(f"oversized split needs {need} bytes", flush=True)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    q, k, v = (t.to(dev) for t in make_qkv(B, H, N, 128, "bf16", 49))
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, N), 7.0, device=dev)
    st = fa.fa_fwd_gen_noalloc(ptr(q), ptr(k), ptr(v), ptr(o), ptr(lse), B, H, N, N, 128, 128,
                               1 / math.sqrt(128), 0, fa.FA_DTYPE_BF16, None, None, stream)
    torch.cuda.synchronize()
    assert st == fa.FA_ERR_SCRATCH
    assert "scratch" in fa.fa_status_string(st)
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())  # nothing written
