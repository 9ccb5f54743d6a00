"""Build the CPU oracle library (test infrastructure only).

    python oracle/build.py        -> oracle/liboasis_oracle.so

Plain gcc, -O2, OpenMP over independent rows; no fast-math, so every double
operation rounds as IEEE-754 prescribes.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oasis_oracle.c")
LIB = os.path.join(HERE, "liboasis_oracle.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
