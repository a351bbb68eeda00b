"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library and never
calls it.  The arithmetic lives in ``oracle.c`` (plain C, fp64); this module
only marshals arrays across ctypes.

What is computed, per row (b, h, i):  the three-pass safe softmax of the scaled
scores ("The Details of Flash Attention", section "Safe Softmax and the Three
Passes") applied to softmax(Q K^T * scale) V ("FlashAttention Engine", the
attention equation), with causal masking keeping key j iff j <= i, and the
per-row log-sum-exp lse = m + ln(l) in natural-log, scaled-score units (the
m and l statistics of "FlashAttention" (ai360xpert), section "Recomputation in
the backward pass").
"""
from __future__ import annotations

import ctypes
import os
import time

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# FA_ORACLE_LIB names another build of the same sources (the sanitizer test)
_LIB_PATH = os.environ.get("FA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

# element-type codes of oracle.h
_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.float64: 3}


def lib():
    """Load liboracle.so (built by oracle/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: run `python oracle/build.py` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_attn_rows.restype = ctypes.c_int
        L.oracle_attn_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_attn_rows_ex.restype = ctypes.c_int
        L.oracle_attn_rows_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_longlong, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_attn_bwd.restype = ctypes.c_int
        L.oracle_attn_bwd.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_double, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_attn_bwd_ex.restype = ctypes.c_int
        L.oracle_attn_bwd_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_longlong, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_attn_rows_gen.restype = ctypes.c_int
        L.oracle_attn_rows_gen.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_attn_bwd_gen.restype = ctypes.c_int
        L.oracle_attn_bwd_gen.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong, ctypes.c_longlong,
            ctypes.c_longlong, ctypes.c_longlong, ctypes.c_double, ctypes.c_int, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_longlong,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.oracle_thread_count.restype = ctypes.c_int
        L.oracle_thread_count.argtypes = [ctypes.c_int]
        L.oracle_load.restype = ctypes.c_double
        L.oracle_load.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong]
        _lib = L
    return _lib


def thread_count(threads: int = 0) -> int:
    return lib().oracle_thread_count(int(threads))


def _as_cpu(t):
    if isinstance(t, np.ndarray):
        t = torch.from_numpy(t)
    if t.device.type != "cpu":
        raise ValueError("the oracle takes host tensors")
    return t.contiguous()


def attn_rows(q, k, v, scale: float, causal: bool, rows=None, threads: int = 0):
    """Oracle attention for selected rows.

    q, k, v: host tensors [B, H, N, d] (float32 / float16 / bfloat16 / float64),
    all of one dtype.  rows: flat row ids (b*H + h)*N + i; None means all rows.
    Returns (o [n_rows, d] float64, lse [n_rows] float64) as numpy arrays.
    """
    q, k, v = _as_cpu(q), _as_cpu(k), _as_cpu(v)
    if not (q.shape == k.shape == v.shape) or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _CODES:
        raise ValueError(f"unsupported dtype combination {q.dtype}/{k.dtype}/{v.dtype}")
    B, H, N, d = q.shape
    if rows is None:
        rows = np.arange(B * H * N, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib().oracle_attn_rows(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _CODES[q.dtype],
        B, H, N, d, float(scale), int(bool(causal)),
        rows.ctypes.data, n, o.ctypes.data, lse.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows failed with code {rc}")
    return o, lse


def attention(q, k, v, scale: float, causal: bool, threads: int = 0):
    """All rows; returns (o [B,H,N,d], lse [B,H,N]) float64 numpy arrays."""
    B, H, N, d = q.shape
    o, lse = attn_rows(q, k, v, scale, causal, None, threads)
    return o.reshape(B, H, N, d), lse.reshape(B, H, N)


def _counts(x, B, name):
    """Per-batch counts as a contiguous int64 array of B entries (or None)."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.cpu().numpy()
    c = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    if c.shape != (B,):
        raise ValueError(f"{name} must hold one count per batch")
    return c


def attn_rows_ex(q, k, v, scale: float, causal: bool, rows=None, k_len=None, threads: int = 0,
                 q_len=None):
    """Oracle attention for query and key sequences of different lengths,
    with optional per-batch valid key counts and a value head dim of its own
    (oracle.h, oracle_attn_rows_gen).

    q: host [B, H, Nq, dk]; k: [B, H, Nk, dk]; v: [B, H, Nk, dv], one dtype.
    rows: flat query-row ids (b*H + h)*Nq + i (None: all).  k_len / q_len: B
    valid key / query counts or None (a query row at or past its batch's count
    is padding and keeps no key).  Returns (o [n_rows, dv], lse [n_rows])
    float64 numpy arrays; rows with no kept key give o = 0, lse = -inf.
    """
    q, k, v = _as_cpu(q), _as_cpu(k), _as_cpu(v)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or k.shape[:3] != v.shape[:3] \
            or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, dk], k [B, H, Nk, dk] and v [B, H, Nk, dv]")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _CODES:
        raise ValueError(f"unsupported dtype combination {q.dtype}/{k.dtype}/{v.dtype}")
    B, H, Nq, dk = q.shape
    Nk, d = k.shape[2], v.shape[3]
    if rows is None:
        rows = np.arange(B * H * Nq, dtype=np.int64)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    kl, ql = _counts(k_len, B, "k_len"), _counts(q_len, B, "q_len")
    n = rows.shape[0]
    o = np.empty((n, d), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rc = lib().oracle_attn_rows_gen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), _CODES[q.dtype], B, H, Nq, Nk, dk, d,
        float(scale), int(bool(causal)), None if kl is None else kl.ctypes.data,
        None if ql is None else ql.ctypes.data,
        rows.ctypes.data, n, o.ctypes.data, lse.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows_gen failed with code {rc}")
    return o, lse


def attention_ex(q, k, v, scale: float, causal: bool, k_len=None, threads: int = 0, q_len=None):
    """All rows of attn_rows_ex; returns (o [B,H,Nq,dv], lse [B,H,Nq])."""
    B, H, Nq, d = q.shape[:3] + v.shape[3:]
    o, lse = attn_rows_ex(q, k, v, scale, causal, None, k_len, threads, q_len)
    return o.reshape(B, H, Nq, d), lse.reshape(B, H, Nq)


def attn_bwd(q, k, v, dout, scale: float, causal: bool, q_rows=None, k_rows=None,
             threads: int = 0):
    """Oracle gradients for selected rows (oracle_bwd.c).

    q, k, v, dout: host tensors [B, H, N, d] of one dtype; dout = dL/dO.
    q_rows / k_rows: flat row ids (b*H + h)*N + i; None means all rows.
    Returns (dq [n_q, d], dk [n_k, d], dv [n_k, d]) float64 numpy arrays.
    """
    q, k, v, dout = _as_cpu(q), _as_cpu(k), _as_cpu(v), _as_cpu(dout)
    if not (q.shape == k.shape == v.shape == dout.shape) or q.dim() != 4:
        raise ValueError("q, k, v, dout must share one [B, H, N, d] shape")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or q.dtype not in _CODES:
        raise ValueError("q, k, v, dout must share one supported dtype")
    B, H, N, d = q.shape
    qr = np.arange(B * H * N, dtype=np.int64) if q_rows is None else q_rows
    kr = np.arange(B * H * N, dtype=np.int64) if k_rows is None else k_rows
    qr = np.ascontiguousarray(np.asarray(qr, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray(kr, dtype=np.int64))
    dq = np.empty((qr.shape[0], d), dtype=np.float64)
    dk = np.empty((kr.shape[0], d), dtype=np.float64)
    dv = np.empty((kr.shape[0], d), dtype=np.float64)
    rc = lib().oracle_attn_bwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), _CODES[q.dtype],
        B, H, N, d, float(scale), int(bool(causal)),
        qr.ctypes.data, qr.shape[0], kr.ctypes.data, kr.shape[0],
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd failed with code {rc}")
    return dq, dk, dv


def attention_bwd(q, k, v, dout, scale: float, causal: bool, threads: int = 0):
    """All rows; returns (dq, dk, dv) [B,H,N,d] float64 numpy arrays."""
    B, H, N, d = q.shape
    dq, dk, dv = attn_bwd(q, k, v, dout, scale, causal, None, None, threads)
    return dq.reshape(B, H, N, d), dk.reshape(B, H, N, d), dv.reshape(B, H, N, d)


def attn_bwd_ex(q, k, v, dout, scale: float, causal: bool, q_rows=None, k_rows=None,
                k_len=None, threads: int = 0, q_len=None):
    """Oracle gradients for unequal lengths, key padding and a value head dim
    of its own (oracle_attn_bwd_gen).

    q: host [B, H, Nq, dk]; k: [B, H, Nk, dk]; v: [B, H, Nk, dv]; dout:
    [B, H, Nq, dv], one dtype.  q_rows: flat ids (b*H + h)*Nq + i; k_rows:
    flat ids (b*H + h)*Nk + j (None: all).  k_len / q_len: B valid key / query
    counts or None.
    Returns (dq [n_q, dk], dk [n_k, dk], dv [n_k, dv]) float64 numpy arrays.
    """
    q, k, v, dout = _as_cpu(q), _as_cpu(k), _as_cpu(v), _as_cpu(dout)
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4 or dout.dim() != 4 \
            or k.shape[:3] != v.shape[:3] or dout.shape != q.shape[:3] + v.shape[3:] \
            or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, dk], k [B, H, Nk, dk], v [B, H, Nk, dv] and "
                         "dout [B, H, Nq, dv]")
    if not (q.dtype == k.dtype == v.dtype == dout.dtype) or q.dtype not in _CODES:
        raise ValueError("q, k, v, dout must share one supported dtype")
    B, H, Nq, d = q.shape
    Nk, d_v = k.shape[2], v.shape[3]
    qr = np.arange(B * H * Nq, dtype=np.int64) if q_rows is None else q_rows
    kr = np.arange(B * H * Nk, dtype=np.int64) if k_rows is None else k_rows
    qr = np.ascontiguousarray(np.asarray(qr, dtype=np.int64))
    kr = np.ascontiguousarray(np.asarray(kr, dtype=np.int64))
    kl, ql = _counts(k_len, B, "k_len"), _counts(q_len, B, "q_len")
    dq = np.empty((qr.shape[0], d), dtype=np.float64)
    dk = np.empty((kr.shape[0], d), dtype=np.float64)
    dv = np.empty((kr.shape[0], d_v), dtype=np.float64)
    rc = lib().oracle_attn_bwd_gen(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), _CODES[q.dtype],
        B, H, Nq, Nk, d, d_v, float(scale), int(bool(causal)),
        None if kl is None else kl.ctypes.data, None if ql is None else ql.ctypes.data,
        qr.ctypes.data, qr.shape[0], kr.ctypes.data, kr.shape[0],
        dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_gen failed with code {rc}")
    return dq, dk, dv


def attention_bwd_ex(q, k, v, dout, scale: float, causal: bool, k_len=None, threads: int = 0,
                     q_len=None):
    """All rows of attn_bwd_ex; returns (dq [B,H,Nq,dk], dk [B,H,Nk,dk],
    dv [B,H,Nk,dv])."""
    B, H, Nq, d = q.shape
    Nk, d_v = k.shape[2], v.shape[3]
    dq, dk, dv = attn_bwd_ex(q, k, v, dout, scale, causal, None, None, k_len, threads, q_len)
    return dq.reshape(B, H, Nq, d), dk.reshape(B, H, Nk, d), dv.reshape(B, H, Nk, d_v)


def timed_attn_rows(q, k, v, scale, causal, rows, threads: int = 0):
    """attn_rows plus the wall time of the C call and the thread count used."""
    nt = min(thread_count(threads), max(1, len(rows)))
    t0 = time.perf_counter()
    o, lse = attn_rows(q, k, v, scale, causal, rows, threads)
    return o, lse, time.perf_counter() - t0, nt
