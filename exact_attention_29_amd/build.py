"""Build libfa.so (the HIP kernels and their C ABI) in-tree for gfx950.

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
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False, resource_usage: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if resource_usage:
        cmd.insert(1, "-Rpass-analysis=kernel-resource-usage")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    noise = ("packed-fp32-ops", "is not a recognized feature for this target")
    err = "\n".join(l for l in res.stderr.splitlines() if not all(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and (verbose or resource_usage):
        print(err)
    os.replace(tmp, LIB)
    return LIB


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
