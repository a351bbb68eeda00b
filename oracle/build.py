"""Build liboracle.so with the host C compiler (no HIP, no GPU headers).

-ffp-contract=off keeps every multiply and add a separately rounded IEEE fp64
operation, so the oracle's arithmetic is exactly what its source says.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def build(verbose: bool = False) -> str:
    out = os.path.join(HERE, "liboracle.so")
    tmp = out + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           os.path.join(HERE, "oracle.c"), os.path.join(HERE, "oracle_bwd.c"), "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
