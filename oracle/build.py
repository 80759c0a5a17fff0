"""Build step for the CPU oracle: gcc -O2 -fopenmp -shared -> oracle/liboracle.so.

Plain -O2 with no -ffast-math, so the C compiler may not reassociate the
oracle's fp64 sums.
"""
from __future__ import annotations

import os
import subprocess

_HERE = os.path.dirname(os.path.abspath(__file__))


def build_oracle(force: bool = True) -> str:
    src = os.path.join(_HERE, "fa_oracle.c")
    out = os.path.join(_HERE, "liboracle.so")
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
