"""Build the oracle's shared library (test infrastructure only).

Compiles oracle.c with the host C compiler into oracle/liboracle.so. Plain IEEE double arithmetic:
no fast-math and no floating-point contraction, so every step rounds as the C source reads.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-Wall", "-Wextra", "-o", LIB + ".tmp",
           os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
