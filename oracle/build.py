"""Compile the C oracle into oracle/libmoe_oracle.so.

TEST INFRASTRUCTURE ONLY.  Strict IEEE arithmetic: -O2, no fast-math, no
floating-point contraction (binary32 products must round one at a time, as
the quantization formula of the CANN "low_latency_dispatch" page states them).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")


def build(verbose=False):
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
        "-Wall", "-Wextra", "-Wno-unused-parameter",
        "-o", LIB + ".tmp", SRC, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
