"""Build the C oracle into oracle/liboracle.so with gcc (test infrastructure).

Flags: -O2 with IEEE binary32 semantics kept intact -- no fast-math, no FMA
contraction (-ffp-contract=off), SSE scalar float on x86-64.  OpenMP only
splits independent rows/blocks, so results do not depend on the thread count.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp4_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fno-strict-aliasing",
          "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force="--lazy" not in sys.argv))
