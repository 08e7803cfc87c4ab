"""CPU oracle for the batch-invariant reductions of an LLM forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.  The
product path (``invariant_amd`` and its HIP library) never imports, links or calls
it, and the two share no code: no kernels, headers, helpers, tables or constants.

Source: the page "Defeating nondeterminism in LLM inference" (Chinese translation),
sections on floating-point non-associativity, batch invariance, RMSNorm, matrix
multiplication and attention; greedy decoding from the page "same LLM, different
GPU, different outputs".

Precision policy
  * fp64 for the GEMM, attention and the decoder layer (graded within 1 bf16 ulp at
    output scale, because the order inside a matrix instruction is the hardware's).
  * exact replay, one IEEE fp32 operation at a time, of the fixed reduction trees of
    RMSNorm and log-softmax (graded bit for bit).  numpy float32 ``+ - * / sqrt`` are
    correctly rounded; ``np.sum``/``np.dot`` are never used to replay a tree because
    they add pairwise/blocked in an order of their own.

Pins (tests/test_oracle_*.py) tie each function to something other than itself:
closed forms, special cases, values printed on the pages, brute force with exact
rational arithmetic on tiny inputs.
"""
from . import fp, check, rmsnorm, logsoftmax, gemm, attention, layer  # noqa: F401
