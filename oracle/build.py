"""Build the CPU oracle (plain C, fp64, OpenMP) with gcc into oracle/liboracle.so.

Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline load the result.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "mla_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
