"""Compile the Conv3D oracle (test infrastructure) into oracle/_conv3d_oracle.so.

The oracle is plain C with OpenMP; it is built for a baseline x86-64-v3 host
so the same shared object runs on any recent x86 machine.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "conv3d_oracle.c")
OUT = os.path.join(HERE, "_conv3d_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
        "-std=c11", "-ffp-contract=off", "-Wall", "-Wextra", "-Wno-unused-parameter",
        SRC, "-o", OUT + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
