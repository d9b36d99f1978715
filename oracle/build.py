"""Builds the CPU oracle (test infrastructure) as oracle/liblq_oracle.so.

Plain gcc, -O2, no fused multiply-add contraction, no fast-math, so every
fp32 codec operation is one IEEE-rounded operation.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "lq_oracle.c")
LIB = os.path.join(HERE, "liblq_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
