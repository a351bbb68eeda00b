"""Benchmark: attention forward TFLOPS and fraction of the MI355X bf16 MFMA peak.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--pass fwd|bwd]

A step is one fa_fwd call (the whole forward pass) over one batch of the
workload, inputs already resident in device memory.  The default workload is
the largest single-GPU one: causal bf16, B=1, H=32, N=65536, d=128, with 1% of
the key rows scaled by 8.  W untimed steps, then K timed steps between two
synchronizations; one JSON line on stdout.  Before every timed step a 1 GiB
device buffer is cleared on the launch stream, outside the step's HIP-event
pair, so that no step starts with the previous step's data in L2 or the
256 MB MALL (--no-flush turns this off).

--pass bwd times the gradients instead: one fa_bwd call (its three kernels)
per step, with the forward outputs O, lse and a seeded dL/dO resident, counted
as 10*B*H*N^2*d algorithmic FLOPs (halved for causal): the five products
S = Q K^T, dV = P^T dO, dP = dO V^T, dQ = dS K and dK = dS^T Q.

Extra objects on the line:
  roofline     -- the kernel's achieved TFLOP/s (algorithmic FLOPs per launch
                  over the mean launch duration from HIP events recorded on
                  the stream the kernel runs on) against the bf16 dense MFMA
                  peak; `traffic` is the HBM bytes per launch measured with
                  rocprofv3 counters, read from the profile summary of the
                  same kernel source (null if the source changed since);
                  `counters` likewise gives the matrix-core busy fraction,
                  the shader clock and the LDS bank-conflict rate from the
                  committed counter summary; `kernel_ms_median` is the median
                  launch beside the mean.
  cpu_baseline -- the fp64 oracle timed on the host cores on a bounded,
                  seeded sample of rows of the same workload, in the same
                  unit; the GPU output on those rows is compared too.

Other modes (used to take the profiles):
  --no-cpu-baseline        skip the oracle leg
  --copy-calibration MiB   run only a plain device copy of that size
  --gemm-reference N       run only a sustained bf16 N x N x N torch.matmul (the
                           vendor GEMM library) and print its TFLOP/s: a
                           practical matrix-core reference on the same box
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS and % of MI355X bf16 MFMA peak (1 GPU)"
METRIC_BWD = "attention bwd TFLOPS and % of MI355X bf16 MFMA peak (1 GPU)"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense
PEAK_FP32_TFLOPS = 157.3    # 256 CU x 256 FLOP/clk x 2.4 GHz, dense MFMA
KERNEL_SRCS = {p: [os.path.join(ROOT, "exact_attention_29_amd", "csrc", n)
                   for n in (f"fa_{p}.hip", "fa_device.h")] for p in ("fwd", "bwd")}


def kernel_source_hash(pass_: str = "fwd") -> str:
    """Hash of one pass's kernel sources (its file and the shared header)."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS[pass_]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_tag(w, pass_: str = "fwd") -> str:
    """Name of what a workload's timed step runs, as used by profiles/: the
    forward kernel instance, or the whole gradient call."""
    if pass_ == "bwd":
        kern = "fa_bwd"  # the whole call: row statistics, dK/dV and dQ kernels
    else:
        kern = "attn_fwd_f32" if w.dtype == "fp32" else "attn_fwd_sp"
    mask = "causal" if w.causal else "noncausal"
    return f"{kern}_{w.dtype}_{mask}_B{w.B}_H{w.H}_N{w.N}_d{w.d}"


def read_traffic(w, pass_: str = "fwd"):
    """HBM bytes per launch from profiles/<kernel tag>.traffic.md, if that
    summary was taken from the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag(w, pass_)}.traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    b = re.search(r"HBM bytes per launch:\s*`?([0-9.eE+]+)", text)
    if not h or not b or h.group(1) != kernel_source_hash(pass_):
        return None
    return float(b.group(1))


def read_counters(w, pass_: str = "fwd"):
    """Matrix-core busy fraction, shader clock and LDS bank-conflict rate from
    profiles/<kernel tag>.counters.md, if taken from the current kernel
    source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag(w, pass_)}.counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    if not h or h.group(1) != kernel_source_hash(pass_):
        return None
    out = {}
    for key, label in (("mfma_busy_frac", "MFMA busy fraction"), ("shader_clock_ghz", "Shader clock GHz"),
                       ("lds_bank_conflict_per_active", "LDS bank-conflict cycles per LDS-active cycle")):
        m = re.search(re.escape(label) + r"[^`]*`([0-9.eE+-]+)`", text)
        out[key] = float(m.group(1)) if m else None
    return out


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size, for scaling the counters."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": 3}))


def gemm_reference(n: int, steps: int = 20) -> None:
    """Sustained throughput of a plain bf16 GEMM through torch (hipBLASLt):
    what the vendor library reaches on dense matrix products on this machine."""
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda", generator=g).to(torch.bfloat16).t().contiguous()
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for e0, e1 in ev:
        e0.record()
        torch.matmul(a, b, out=c)
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    tf = 2.0 * n ** 3 / ms / 1e9
    print(json.dumps({"gemm_reference": f"bf16 {n}x{n}x{n} torch.matmul", "ms": round(ms, 4),
                      "tflops": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                      "steps": steps}))


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or 'unknown'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, q, k, v, o_gpu, lse_gpu, target_s: float, seed: int = 0):
    """Time the oracle on a seeded uniform sample of rows sized to ~target_s."""
    import oracle

    rng = np.random.default_rng(seed)
    total_rows = w.B * w.H * w.N

    def flops(rows):
        pos = rows % w.N
        keys = (pos + 1) if w.causal else np.full_like(pos, w.N)
        return float((4.0 * keys * w.d).sum())

    perm = rng.permutation(total_rows)
    first = np.sort(perm[:min(512, total_rows)])
    o1, l1, t1, nt = oracle.timed_attn_rows(q, k, v, w.scale, w.causal, first)
    rate = flops(first) / max(t1, 1e-9)
    # enough further rows to bring the total to about target_s
    avg = flops(first) / len(first)
    more = int(max(0.0, target_s - t1) * rate / avg)
    more = min(more, total_rows - len(first))
    rows, o_ref, l_ref, secs = first, o1, l1, t1
    if more > 0:
        second = np.sort(perm[len(first):len(first) + more])
        o2, l2, t2, _ = oracle.timed_attn_rows(q, k, v, w.scale, w.causal, second)
        rows = np.concatenate([first, second])
        o_ref, l_ref, secs = np.concatenate([o1, o2]), np.concatenate([l1, l2]), t1 + t2
    fl = flops(rows)
    og = o_gpu.double().cpu().reshape(total_rows, w.d).numpy()[rows]
    lg = lse_gpu.double().cpu().reshape(total_rows).numpy()[rows]
    parity = {"rows": int(len(rows)), "max_abs_o": float(np.abs(og - o_ref).max()),
              "mean_abs_o": float(np.abs(og - o_ref).mean()),
              "max_abs_lse": float(np.abs(lg - l_ref).max())}
    return {
        "value": fl / secs / 1e12, "unit": "TFLOPS", "cores": int(nt), "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"{len(rows)} of {total_rows} query rows of the workload, seeded uniform "
                   f"over batch, head and position; FLOPs counted 4*|keys kept|*d per row; "
                   f"{secs:.1f} s of oracle time"),
        "seconds": secs, "gflop": fl / 1e9,
    }, parity


def cpu_baseline_bwd(w, q, k, v, g, dq, dk, dv, target_s: float):
    """Time the gradient oracle on whole heads of the workload (as many as fit
    about target_s, at least one), in the same algorithmic-FLOP unit."""
    import oracle

    B, H, N, d = w.B, w.H, w.N, w.d
    per_head = 10.0 * N * N * d / (2.0 if w.causal else 1.0)
    heads, secs, errs = 0, 0.0, []
    nt = oracle.thread_count(0)
    for idx in range(B * H):
        b, h = divmod(idx, H)
        rows = np.arange(idx * N, (idx + 1) * N, dtype=np.int64)
        t0 = time.perf_counter()
        rq, rk, rv = oracle.attn_bwd(q, k, v, g, w.scale, w.causal, rows, rows)
        secs += time.perf_counter() - t0
        heads += 1
        for got, ref in ((dq, rq), (dk, rk), (dv, rv)):
            x = got[b, h].double().cpu().numpy()
            errs.append(float(np.abs(x - ref).max()) / max(float(np.abs(ref).max()), 1e-2))
        if secs >= target_s:
            break
    return {
        "value": heads * per_head / secs / 1e12, "unit": "TFLOPS", "cores": int(nt),
        "kind": "oracle", "cpu_model": cpu_model(),
        "sample": (f"all rows of {heads} of {B * H} heads of the workload (dq, dk, dv), FLOPs "
                   f"counted 10*N^2*d per head{' halved for causal' if w.causal else ''}; "
                   f"{secs:.1f} s of oracle time"),
        "seconds": secs, "gflop": heads * per_head / 1e9,
    }, {"heads": heads, "max_abs_over_max_ref": max(errs)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-flush", action="store_true",
                    help="do not clear a 1 GiB buffer before each timed step")
    ap.add_argument("--pass", dest="pass_", choices=["fwd", "bwd"], default="fwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB")
    ap.add_argument("--gemm-reference", type=int, default=0, metavar="N")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build runs the forward pass on a single "
              "MI355X (no sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        return 1
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    if args.gemm_reference:
        gemm_reference(args.gemm_reference, args.steps)
        return 0

    import exact_attention_29_amd as fa
    from exact_attention_29_amd.inputs import WORKLOADS, make_dout, workload_inputs

    w = WORKLOADS[args.workload]
    bwd = args.pass_ == "bwd"
    if bwd and not fa.fa_bwd_supported(w.d, fa.FA_DTYPE_BF16 if w.dtype == "bf16" else
                                       fa.FA_DTYPE_FP16 if w.dtype == "fp16" else fa.FA_DTYPE_FP32,
                                       int(w.causal)):
        print(f"no gradient kernels for workload {args.workload} ({w.dtype}, d={w.d})",
              file=sys.stderr)
        return 1
    q_h, k_h, v_h = workload_inputs(w)
    dev = torch.device("cuda:0")
    q, k, v = q_h.to(dev), k_h.to(dev), v_h.to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if bwd:
        g_h = make_dout(w.B, w.H, w.N, w.d, w.dtype, 100 + args.workload)
        g = g_h.to(dev)
        fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))

        def step():
            fa.attention_bwd(q, k, v, o, lse, g, causal=w.causal, scale=w.scale, dq=dq, dk=dk,
                             dv=dv, stream=stream)
        flops = 2.5 * w.flops
    else:
        def step():
            fa.attention(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        flops = w.flops

    # L2 and MALL eviction between timed steps: clearing 1 GiB (4x the MALL)
    # on the launch stream, outside each step's event pair
    flush_buf = None if args.no_flush else torch.empty(1 << 28, dtype=torch.float32, device=dev)

    def flush():
        if flush_buf is not None:
            with torch.cuda.stream(stream):
                flush_buf.zero_()

    for _ in range(args.warmup):
        flush()
        step()
    torch.cuda.synchronize(dev)

    # timed region: K steps; a HIP event pair around every step on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for a, b in ev:
        flush()
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    per_launch = [a.elapsed_time(b) for a, b in ev]
    kernel_ms = float(np.mean(per_launch))

    # the step time is the event-timed step (the flush between steps is not
    # part of the step); the wall time of the whole timed loop, flushes
    # included, is reported beside it
    ms_per_step = kernel_ms if flush_buf is not None else wall * 1e3 / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype in ("bf16", "fp16") else PEAK_FP32_TFLOPS
    traffic = read_traffic(w, args.pass_)
    elem = 2 if w.dtype != "fp32" else 4
    if bwd:  # read Q, K, V, O, dO, lse; write dQ, dK, dV
        algo_bytes = 8 * w.B * w.H * w.N * w.d * elem + 4 * w.B * w.H * w.N
    else:    # read Q, K, V; write O, lse
        algo_bytes = 4 * w.B * w.H * w.N * w.d * elem + 4 * w.B * w.H * w.N
    line = {
        "metric": METRIC_BWD if bwd else METRIC, "value": round(value, 2), "unit": "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) per the workload recipe)",
        "config": {**w.as_dict(), "pass": args.pass_, "flops_per_step": flops,
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "l2_mall_flush_between_steps": flush_buf is not None,
                   "wall_ms_per_step_incl_flush": round(wall * 1e3 / args.steps, 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel_ms": round(kernel_ms, 4),
                     "kernel_ms_median": round(float(np.median(per_launch)), 4),
                     "counters": read_counters(w, args.pass_),
                     "algorithmic_bytes": algo_bytes,
                     "kernel_source_sha256_16": kernel_source_hash(args.pass_)},
    }
    if bwd:
        line["roofline"]["timed"] = "whole fa_bwd call (row statistics, dK/dV and dQ kernels)"
    if not args.no_cpu_baseline:
        if bwd:
            cb, par = cpu_baseline_bwd(w, q_h, k_h, v_h, g_h, dq, dk, dv, args.cpu_seconds)
        else:
            cb, par = cpu_baseline(w, q_h, k_h, v_h, o, lse, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity_on_cpu_sample"] = par
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
