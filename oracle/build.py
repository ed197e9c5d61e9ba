"""Build the CPU oracle (test infrastructure; never part of the product path).

Compiles oracle.c with gcc into liboracle.so next to this file.  Plain loops,
OpenMP across output rows, and -ffp-contract=off so that the epilogue's
multiplies are each rounded on their own.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build_oracle(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
