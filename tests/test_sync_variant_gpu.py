"""Race check of the pipelined forward kernels: libfa_sync.so is the same
source built with FA_SYNC_PHASES, in which every tile's loads complete (and,
in the 16-bit kernel, the whole workgroup meets at a barrier) before any wave
reads the tile, and barriers surround each epilogue staging phase.  Its
arithmetic is the same, so on every shape its O and lse must equal
libfa.so's bit for bit; a load that the pipelined kernel read too early, or a
stage buffer overwritten while still being read, would show as a difference.
Both libraries are called through the C ABI.
"""
import ctypes
import math
import os

import pytest
import torch

import exact_attention_29_amd as fa
from exact_attention_29_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(fa.__file__))
DT = {"bf16": (torch.bfloat16, fa.FA_DTYPE_BF16), "fp16": (torch.float16, fa.FA_DTYPE_FP16),
      "fp32": (torch.float32, fa.FA_DTYPE_FP32)}


@pytest.fixture(scope="module")
def sync_lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU; run with -m 'not gpu' on a CPU host"
    path = os.path.join(HERE, "libfa_sync.so")
    assert os.path.exists(path), f"{path} is not built (python -m exact_attention_29_amd.build)"
    L = ctypes.CDLL(path)
    L.fa_fwd_gen.restype = ctypes.c_int
    L.fa_fwd_gen.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + [
        ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.fa_fwd_gen_workspace_size.restype = ctypes.c_size_t
    L.fa_fwd_gen_workspace_size.argtypes = [ctypes.c_int] * 8
    return L


CASES = [
    # (dt, B, H, Nq, Nk, dk, dv, causal, k_len, q_len, split)
    ("bf16", 4, 32, 2048, 2048, 64, 64, False, None, None, False),     # workload 3's shape
    ("bf16", 2, 32, 8192, 8192, 128, 128, True, None, None, False),    # workload 4's shape
    ("bf16", 2, 8, 1000, 1500, 128, 128, True, [1500, 777], [1000, 433], False),
    ("fp16", 3, 5, 891, 891, 64, 64, True, None, None, False),
    ("bf16", 1, 4, 4096, 4096, 128, 128, True, None, None, True),      # key split
    ("fp16", 2, 2, 700, 2300, 64, 128, False, [2300, 1111], None, True),
    # fp32: K tiles loaded into LDS behind the products, V rows into registers
    ("fp32", 1, 1, 1024, 1024, 1024, 1024, False, None, None, True),  # the wide-head shape, key split
    ("fp32", 2, 3, 333, 1000, 512, 512, True, [1000, 457], [333, 100], False),
    ("fp32", 2, 4, 1500, 1500, 128, 128, True, None, None, False),
    ("fp32", 3, 2, 777, 901, 64, 128, False, [901, 13], None, True),
    ("fp32", 2, 2, 300, 300, 128, 64, True, [300, 299], [300, 31], False),
    ("fp32", 1, 2, 391, 391, 128, 128, True, None, None, True),     # two waves of 64 columns, key split
    ("fp32", 2, 2, 500, 700, 256, 256, False, [700, 350], None, True),  # four waves of 64 columns
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-B{c[1]}H{c[2]}Nq{c[3]}Nk{c[4]}d{c[5]}x{c[6]}"
                                              f"{'-causal' if c[7] else ''}{'-split' if c[10] else ''}"
                                              for c in CASES])
def test_synchronised_build_matches_bitwise(sync_lib, case):
    dt, B, H, Nq, Nk, dk, dv, causal, k_len, q_len, split = case
    print(f"case {case}", flush=True)
    tdt, code = DT[dt]
    q, k, _ = make_qkv(B, H, max(Nq, Nk), dk, dt, seed=91)
    _, _, v = make_qkv(B, H, Nk, dv, dt, seed=92)
    dev = torch.device("cuda")
    q = q[:, :, :Nq].contiguous().to(dev)
    k = k[:, :, :Nk].contiguous().to(dev)
    v = v.to(dev)
    kl = None if k_len is None else torch.tensor(k_len, dtype=torch.int32, device=dev)
    ql = None if q_len is None else torch.tensor(q_len, dtype=torch.int32, device=dev)
    scale = 1 / math.sqrt(dk)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for lib in (fa.library(), sync_lib):
        o = torch.full((B, H, Nq, dv), float("nan"), dtype=tdt, device=dev)
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=dev)
        ws_bytes = lib.fa_fwd_gen_workspace_size(B, H, Nq, Nk, dk, dv, int(causal), code) if split else 0
        assert (ws_bytes > 0) == split
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        st = lib.fa_fwd_gen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, H, Nq, Nk, dk, dv, ctypes.c_float(scale), int(causal), code,
                            None if kl is None else kl.data_ptr(),
                            None if ql is None else ql.data_ptr(),
                            ws.data_ptr() if ws_bytes else None, ws_bytes, stream)
        assert st == fa.FA_OK, fa.fa_status_string(st)
        outs.append((o, lse))
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = outs
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
