"""GPU checks of the persistent work distribution at head dim 128 (bf16, fp16):
one workgroup per compute unit claims (query block, head) items until none is
left, so every item must be claimed exactly once even when many items have no
key tile to run -- blocks of padding rows (q_len), batches with no valid key
(k_len = 0), and causal blocks that lie wholly before the first key when
there are more queries than keys.  Every shape here has far more items than
the GPU has compute units.

The outputs are filled with NaN before each call: an item that no workgroup
ran would leave NaN behind.  Rows that keep no key must be exactly O = 0,
lse = -inf (the empty sum); sampled rows with keys are compared with the fp64
oracle within the workload tolerance.
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
DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def kept_rows(B, H, Nq, Nk, q_len, k_len, causal):
    """Boolean [B, H, Nq]: rows that keep at least one key (the rule of the
    C header: row i < Lq keeps key j iff j < L and, causal, j <= i + L - Lq)."""
    keep = np.zeros((B, H, Nq), dtype=bool)
    for b in range(B):
        L = Nk if k_len is None else min(max(k_len[b], 0), Nk)
        Lq = Nq if q_len is None else min(max(q_len[b], 0), Nq)
        i = np.arange(Nq)
        ok = (i < Lq) & (L > 0)
        if causal:
            ok &= i + (L - Lq) >= 0
        keep[b, :, :] = ok[None, :]
    return keep


CASES = [
    # (B, H, Nq, Nk, q_len, k_len, causal, dtype)
    (2, 32, 8192, 8192, [8192, 1024], None, False, "bf16"),   # 896 of 2048 blocks padding
    (1, 64, 8192, 1024, None, None, True, "bf16"),           # 1792 of 2048 blocks before key 0
    (2, 32, 4096, 4096, None, [0, 4096], False, "bf16"),     # a batch without keys
    (2, 32, 4096, 4096, [4096, 300], [0, 2000], True, "bf16"),
    (2, 32, 4096, 4096, [4096, 513], None, True, "fp16"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}H{c[1]}Nq{c[2]}Nk{c[3]}q{c[4]}k{c[5]}"
                                              f"{'c' if c[6] else 'n'}-{c[7]}" for c in CASES])
def test_every_item_claimed(case):
    B, H, Nq, Nk, q_len, k_len, causal, dt = case
    d = 128
    print(f"case {case}", flush=True)
    q, k, v = make_qkv(B, H, max(Nq, Nk), d, dt, seed=601)
    q, k, v = q[:, :, :Nq].contiguous(), k[:, :, :Nk].contiguous(), v[:, :, :Nk].contiguous()
    scale = 1 / math.sqrt(d)
    dev = torch.device("cuda")
    out = torch.full((B, H, Nq, d), float("nan"), dtype=DT[dt], device=dev)
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
    ql = None if q_len is None else torch.tensor(q_len, dtype=torch.int32, device=dev)
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device=dev)
    fa.attention(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale, out=out, lse=lse,
                 k_len=kl, q_len=ql)
    torch.cuda.synchronize()
    og = out.double().cpu().numpy()
    lg = lse.double().cpu().numpy()
    keep = kept_rows(B, H, Nq, Nk, q_len, k_len, causal)
    assert not np.isnan(og).any() and not np.isnan(lg).any(), "an item was never run"
    assert np.all(og[~keep] == 0) and np.all(np.isneginf(lg[~keep])), "rows without keys"
    assert np.isfinite(og[keep]).all() and np.isfinite(lg[keep]).all()
    # sampled rows with keys against the oracle: the first, last and a random
    # row of every (b, h), plus random rows over the whole output
    rng = np.random.default_rng(5)
    flat = np.flatnonzero(keep.reshape(-1))
    pick = set(rng.choice(flat, size=min(600, flat.size), replace=False).tolist())
    for bh in range(B * H):
        rows_bh = flat[(flat >= bh * Nq) & (flat < (bh + 1) * Nq)]
        if rows_bh.size:
            pick.update((int(rows_bh[0]), int(rows_bh[-1])))
    rows = np.array(sorted(pick), dtype=np.int64)
    o_ref, l_ref = oracle.attn_rows_ex(q, k, v, scale, causal, rows, k_len, q_len=q_len)
    do = np.abs(og.reshape(-1, d)[rows] - o_ref)
    dl = np.abs(lg.reshape(-1)[rows] - l_ref)
    st = dict(max_o=float(do.max()), mean_o=float(do.mean()), max_lse=float(dl.max()),
              rows=int(rows.size), finite=True)
    print(st)
    parity.check(st, DT[dt])
