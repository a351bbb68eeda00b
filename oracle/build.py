"""Build liboracle.so with the host C compiler (no HIP, no GPU headers).

-ffp-contract=off keeps every multiply and add a separately rounded IEEE fp64
operation, so the oracle's arithmetic is exactly what its source says.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


# AddressSanitizer + UndefinedBehaviorSanitizer build (test runs only): ROCm's
# clang, whose shared sanitizer runtime also serves the host-sanitized libfa
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all", "-shared-libsan"]
CLANG = "/opt/rocm/llvm/bin/clang"


def build(verbose: bool = False, sanitize: bool = False, out: str = "", src_dir: str = "") -> str:
    """Build liboracle.so in this directory (or at `out`) from the sources here
    (or in `src_dir`); with sanitize, instrumented with ASan and UBSan."""
    out = out or os.path.join(HERE, "liboracle.so")
    src = src_dir or HERE
    tmp = out + ".tmp"
    cc, opt = (CLANG, SANITIZE_FLAGS) if sanitize else ("gcc", ["-O2"])
    cmd = [cc, "-std=c11", *opt, "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           os.path.join(src, "oracle.c"), os.path.join(src, "oracle_bwd.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
