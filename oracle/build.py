"""Compile the C oracle into oracle/libdcnv4_oracle.so (test infrastructure).

Strict IEEE binary32 semantics: no contraction except the explicit fmaf calls,
no fast-math, no vector ISA assumptions beyond the x86-64 baseline.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "dcnv4_oracle.c")
LIB = os.path.join(HERE, "libdcnv4_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fno-strict-aliasing", "-Wall", "-Wextra", "-shared", "-fPIC",
           "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
