"""Build the CPU oracle shared library (plain C, gcc, OpenMP).

Test infrastructure only: the product path never loads what this builds.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRCS = [os.path.join(HERE, "lbsa_oracle.c"), os.path.join(HERE, "prologue_oracle.c")]
LIB = os.path.join(HERE, "liblbsa_oracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle's C sources into oracle/liblbsa_oracle.so and return its path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           "-Wall", "-Wextra", "-Wno-unused-parameter", *SRCS, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
