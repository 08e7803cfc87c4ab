"""Build tests/c/gemm_from_c (a plain C program driving the library through include/bi.h
with HIP-runtime device memory) with gcc, linked to invariant_amd/libbi.so and the HIP
runtime; test-only.

    python -m tests.c.build        # also run by __graft_entry__.build()
"""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(HERE, "gemm_from_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        raise RuntimeError("no C compiler for tests/c")
    libdir = os.path.join(ROOT, "invariant_amd")
    tmp = OUT + ".tmp"
    cmd = [cc, "-std=c99", "-O2", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "gemm_from_c.c"), "-o", tmp,
           f"-L{libdir}", "-l:libbi.so", f"-L{os.path.join(ROCM, 'lib')}", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../invariant_amd", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building tests/c/gemm_from_c failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
