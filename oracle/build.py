"""Build the oracle's C pieces in place (TEST INFRASTRUCTURE: only tests/ load them).

    python -m oracle.build

oracle/libexplog.so -- the C replay of the oracle's EXP and LOG (explog.c), for the
exhaustive sweeps of the GPU's functions.  Plain gcc, IEEE binary32 arithmetic with no
contraction of multiply-adds and no fast-math.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "libexplog.so")


def build() -> str:
    tmp = OUT + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", os.path.join(HERE, "explog.c"), "-o", tmp], check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
