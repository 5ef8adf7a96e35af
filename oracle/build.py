"""Compile the CPU oracle (plain C) into oracle/liboracle.so with gcc.

Test infrastructure: the oracle is built so that the tests, the smoke check
and the benchmark's CPU-baseline leg can run it.  Strict IEEE arithmetic: no
fast-math, no FMA contraction.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra", "-Wno-unused-parameter",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
