"""Build libfa.so (the HIP kernels and their C ABI) in-tree for gfx950, and
libfa_sync.so, the forward's synchronised check build.

    python -m exact_attention_29_amd.build [-v] [--resource-usage]

Flags: -O3 for gfx950 only; packed-fp32 instructions are switched off
(-packed-fp32-ops) so the compiler emits only scalar fp32 VALU operations.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", n) for n in ("fa_fwd.hip", "fa_bwd.hip")]
LIB = os.path.join(HERE, "libfa.so")
# the forward built with FA_SYNC_PHASES: a barrier before every tile's LDS
# reads (checked bitwise against libfa.so by the GPU tests; never the product)
LIB_SYNC = os.path.join(HERE, "libfa_sync.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    """Build libfa.so and its synchronised check build libfa_sync.so (two
    hipcc processes side by side)."""
    jobs = [_start(LIB, SOURCES, [], verbose, resource_usage),
            _start(LIB_SYNC, SOURCES[:1], ["-DFA_SYNC_PHASES"], verbose, False)]
    for lib, proc in jobs:
        _finish(lib, proc, verbose or resource_usage)
    return LIB


def _start(lib: str, sources, defines, verbose: bool, resource_usage: bool):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *defines,
           "-I", os.path.join(ROOT, "include"), *sources, "-o", lib + ".tmp"]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    return lib, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(lib: str, proc, show: bool) -> None:
    _, stderr = proc.communicate()
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    err = "\n".join(l for l in stderr.splitlines() if not all(n in l for n in noise))
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}) for {os.path.basename(lib)}:\n{err}")
    if err.strip() and show:
        print(err)
    os.replace(lib + ".tmp", lib)


def build_host_sanitized(out: str, verbose: bool = False) -> str:
    """libfa.so with its host half (argument checks, planning, the C ABI)
    instrumented with AddressSanitizer and UndefinedBehaviorSanitizer, for the
    CPU-only sanitizer test; the device code is built as usual.  Uses the
    shared clang sanitizer runtime."""
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-shared", "-fPIC",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Xarch_host", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-Xarch_host", "-shared-libsan", "-Xarch_host",
           "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, resource_usage="--resource-usage" in sys.argv))
