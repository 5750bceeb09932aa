"""Builds the C oracle (test infrastructure) into oracle/_build/libsage_oracle.so.

Plain gcc, -O2, OpenMP, no FMA contraction, no fast-math: every binary32
operation in the source is rounded exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "sage_oracle.c")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libsage_oracle.so")

CFLAGS = [
    "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
    "-fexcess-precision=standard", "-fPIC", "-shared", "-Wall", "-Wextra",
]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
