"""Builds the CPU oracle library ``libugref.so`` from ``ugref.c`` with gcc.

Test infrastructure only: the oracle is built so that tests, the smoke check
and the benchmark's CPU baseline can run it.  The flags keep every float
operation a single binary32 operation: no FMA contraction, no fast-math, no
flush-to-zero (x86-64 SSE arithmetic, no x87 extended precision).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ugref.c")
LIB = os.path.join(HERE, "libugref.so")

CFLAGS = [
    "-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-fexcess-precision=standard",
    "-Wall", "-Wextra",
]


def build(force: bool = True) -> str:
    """Compile the oracle; returns the library path."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
