"""Builds the oracle's shared library with the host C compiler.

The oracle is test infrastructure (see ``oracle/__init__.py``). Plain fp64 C, no
fast-math and no FMA contraction, so each operation is one IEEE rounding in the order
the source writes it.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rgdr_oracle.c")
LIB = os.path.join(HERE, "librgdr_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
