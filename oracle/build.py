"""Build ``oracle/liboracle.so`` with the host C compiler (test infrastructure only).

Plain C, -O2, no fast-math and no vector intrinsics, so that the fp64 sums keep
IEEE semantics in program order.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")


def build() -> str:
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-pthread", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
