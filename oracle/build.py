"""Compile the C oracle into oracle/_build/libw8oracle.so.

Test infrastructure only (see oracle/__init__.py).  The flags matter for the
oracle's arithmetic: no -ffast-math and no floating-point contraction, so that
float division and nearbyint() are the IEEE-754 operations the oracle's
definitions name.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "w8_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libw8oracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
          "-ffp-contract=off", "-std=c11", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
