"""Build the CPU oracle library (test infrastructure only).

Compiles ``oracle.c`` with gcc into ``liboracle.so`` next to this file.
Floating-point contraction is disabled so that every product and every sum
of the reference is rounded separately.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
           "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra", "-Wno-unused-parameter",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
