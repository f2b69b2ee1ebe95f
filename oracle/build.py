"""Build the CPU oracle (test infrastructure) with gcc.

The oracle is plain C with no dependency on the GPU library: it is compiled
here on its own, into ``oracle/liboracle.so``.  ``-ffp-contract=off`` keeps the
binary64 multiply and add separate (no fused multiply-add), so every output is
the same sequential sum on any host.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
