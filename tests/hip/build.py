"""Build the test-only HIP library tests/hip/libfpsweep.so (exhaustive sweeps of the
library's contract fp32 functions) with the product library's compiler flags.

    python -m tests.hip.build        # also run by __graft_entry__.build()
"""
from __future__ import annotations

import os

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "libfpsweep.so")


def build() -> str:
    from invariant_amd.build import FLAGS, HIPCC, _run
    tmp = OUT + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", os.path.join(HERE, "fpsweep.hip"), "-o", tmp])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
