"""Compile the C oracle into ``oracle/liboracle_topk.so`` (test infrastructure only).

Run as ``python oracle/build.py`` or call :func:`build`. Uses the host gcc with
OpenMP; nothing here is GPU code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "topk_sort.c")
LIB = os.path.join(HERE, "liboracle_topk.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra",
           SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
