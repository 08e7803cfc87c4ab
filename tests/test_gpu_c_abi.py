"""The library driven from a plain C program with HIP-runtime device memory and no torch
(tests/c/gemm_from_c.c, built by __graft_entry__.build()): integer-valued GEMM operands
make the expected outputs exact, so the check is bit for bit (fp32 output = the integer
product, bf16 output = its one RNE rounding, a one-row call = the full call's row, argmax
of rows with a unique maximum = its index)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "gemm_from_c")


def test_plain_c_program_on_the_gpu():
    if not os.path.exists(EXE):
        raise RuntimeError("tests/c/gemm_from_c is not built: run __graft_entry__.build()")
    print("c-abi: tests/c/gemm_from_c (300 x 257 x 1000 GEMM, 3-row argmax)", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
