"""Build the oracle's shared library with gcc (plain C99 + OpenMP).

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "k3moe_oracle.c")
LIB = os.path.join(HERE, "libk3oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-semantic-interposition", "-Wall", "-Wextra", "-o", LIB, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
