"""Build the CPU oracle (test infrastructure only) into oracle/liboracle.so.

Plain g++, one translation unit, no OpenMP, no BLAS, no FP contraction and no
fast-math, so every dot product runs as written in moe_oracle.cc.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "moe_oracle.cc")
    tmp = LIB + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-o", tmp, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
