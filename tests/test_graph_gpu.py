"""HIP graph capture of the forward and gradient calls (bf16, and fp32 at
d = 1024 and with per-batch counts): each captured call
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


@pytest.mark.parametrize("dt,B,H,N,d,causal,counts", [
    ("bf16", 2, 8, 1024, 128, True, False),    # persistent forward
    ("bf16", 1, 2, 4096, 128, False, False),   # key split of the 16-bit forward
    ("bf16", 2, 4, 700, 64, True, False),      # one workgroup per block (d = 64)
    ("bf16", 2, 4, 900, 128, True, True),      # per-batch key and query counts
    ("fp32", 1, 1, 1024, 1024, False, False),  # fp32 wide heads: eight waves, key split
    ("fp32", 2, 3, 600, 128, True, True),      # fp32 with per-batch counts
])
def test_captured_calls_replay_bitwise(dt, B, H, N, d, causal, counts):
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, dt, 31 + N))
    g = make_dout(B, H, N, d, dt, 32 + N).cuda()
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


def test_shared_counter_slot_concurrent_replays():
    """Two captured calls that hold the same counter slot of the persistent
    forward (the host hands out 64 slots round-robin; the second capture comes
    64 calls after the first) replayed at the same time on two streams, next to
    eager calls on a third: each writes its own outputs, and every output must
    equal the eager result bit for bit.  A launch that finds its slot held by
    another launch runs its items in its own static order instead."""
    B, H, N, d = 1, 32, 16384, 128
    q, k, v = (t.cuda() for t in make_qkv(B, H, N, d, "bf16", 77))
    o_ref, l_ref = fa.attention(q, k, v, causal=True)
    torch.cuda.synchronize()
    outs = [(torch.empty_like(o_ref), torch.empty_like(l_ref)) for _ in range(3)]
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    graphs = []
    for gi in range(2):
        o, lse = outs[gi]
        s1.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            fa.attention(q, k, v, causal=True, out=o, lse=lse)  # warm-up call on the side stream
        torch.cuda.current_stream().wait_stream(s1)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fa.attention(q, k, v, causal=True, out=o, lse=lse)
        graphs.append(g)
        if gi == 0:
            # 62 calls of the same kernel, then the next warm-up call: the
            # second capture is the 64th call after the first and draws its slot
            for _ in range(62):
                fa.attention(q, k, v, causal=True, out=outs[2][0], lse=outs[2][1])
            torch.cuda.synchronize()
    for rep in range(6):
        for o, lse in outs:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        with torch.cuda.stream(s2):
            graphs[1].replay()
        with torch.cuda.stream(s3):
            for _ in range(3):
                fa.attention(q, k, v, causal=True, out=outs[2][0], lse=outs[2][1])
        torch.cuda.synchronize()
        for i, (o, lse) in enumerate(outs):
            assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), (rep, i)
    # the same captured call replayed on two streams without a sync between
    for rep in range(3):
        outs[0][0].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        with torch.cuda.stream(s2):
            graphs[0].replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0][0], o_ref) and torch.equal(outs[0][1], l_ref), rep
