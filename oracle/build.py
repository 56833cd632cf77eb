"""Compile the C oracle into oracle/liboracle.so (plain gcc, no fast-math, no FMA contraction)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "vbq_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB_PATH, extra=()) -> str:
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
