"""Compile the CPU oracle (plain C, gcc) into oracle/liboracle_mx.so.

Test infrastructure: building the checker is not using it.  Flags keep
IEEE semantics: no fast-math, no FMA contraction, SSE fp32 arithmetic.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_mx.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "mx_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fexcess-precision=standard", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
