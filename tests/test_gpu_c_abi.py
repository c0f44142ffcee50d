"""The C ABI from plain C on the GPU: tests/c/mm_from_c (built by
__graft_entry__.build()) runs linear + bias + GELU, the SwiGLU FFN and an
fp32 NN matmul through include/mm.h with memory from the HIP runtime's C API,
and compares every output with the oracle's C library.  It runs as a child
process of its own."""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "mm_from_c")


def test_c_program_gemm_matches_oracle():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "tests/c/mm_from_c is not built (run __graft_entry__.build())"
    print("case: C program gemm", flush=True)
    r = subprocess.run([EXE, "gemm"], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")
