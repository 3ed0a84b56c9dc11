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


# Sanitizer builds (test infrastructure): liboracle_ubsan.so, loaded by
# oracle/ref.py when FP4Q_SANITIZE=1, and an ASan + UBSan executable from a C
# driver linked with the oracle's source.
LIB_UBSAN = os.path.join(HERE, "liboracle_ubsan.so")
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def build_ubsan() -> str:
    tmp = LIB_UBSAN + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, *SAN_FLAGS, "-fsanitize=undefined", SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, LIB_UBSAN)
    return LIB_UBSAN


def build_asan_driver(driver: str, out: str) -> str:
    flags = [f for f in CFLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run(["gcc", *flags, *SAN_FLAGS, "-fsanitize=address,undefined", SRC, driver, "-o", out, "-lm"],
                   check=True)
    return out


if __name__ == "__main__":
    if "--ubsan" in sys.argv:
        print(build_ubsan())
    else:
        print(build(force="--lazy" not in sys.argv))
