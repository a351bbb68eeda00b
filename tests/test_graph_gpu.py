"""HIP graph capture of the forward and gradient calls: each captured call
replays several times, with other eager work and synchronisations between
the replays, and every replay must equal the eager result bit for bit (the
persistent forward resets its work counters at the end of each launch, the
key split and the gradients use a workspace from torch's graph pool).
"""
import pytest
import torch

import exact_attention_29_amd as fa
from exact_attention_29_amd.inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("B,H,N,d,causal,counts", [
    (2, 8, 1024, 128, True, False),    # persistent forward
    (1, 2, 4096, 128, False, False),   # key split of the 16-bit forward
    (2, 4, 700, 64, True, False),      # one workgroup per block (d = 64)
    (2, 4, 900, 128, True, True),      # per-batch key and query counts
])
def test_captured_calls_replay_bitwise(B, H, N, d, causal, counts):
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, "bf16", 31 + N))
    g = make_dout(B, H, N, d, "bf16", 32 + N).cuda()
    kw = dict(causal=causal)
    if counts:
        kw.update(k_len=torch.tensor([N, N // 3], dtype=torch.int32, device="cuda"),
                  q_len=torch.tensor([N // 2, N], dtype=torch.int32, device="cuda"))
    # eager reference
    o_ref, l_ref = fa.attention(q, k, v, **kw)
    dq_ref, dk_ref, dv_ref = fa.attention_bwd(q, k, v, o_ref, l_ref, g, **kw)
    torch.cuda.synchronize()
    # capture (warm the side stream first, as torch recommends)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, lse = fa.attention(q, k, v, **kw)
        fa.attention_bwd(q, k, v, o, lse, g, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o, lse = fa.attention(q, k, v, **kw)
        dq, dk, dv = fa.attention_bwd(q, k, v, o, lse, g, **kw)
    for rep in range(4):
        for t in (o, lse, dq, dk, dv):
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
        assert torch.equal(dq, dq_ref) and torch.equal(dk, dk_ref) and torch.equal(dv, dv_ref), rep
