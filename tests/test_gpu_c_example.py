"""The plain C caller of the library (csrc/example_c.c, built beside
libsolattn.so): run as its own process with no Python in the loop, it pools,
routes and attends at tau = 8 and tau = +inf through the C ABI and checks a
few rows of the dense result against softmax attention in double precision
(max abs error 2e-2, the same bar as the bf16 parity tests' largest cases).
"""
import os
import subprocess

import pytest
import torch

import block_sparse_attention_14_amd as sa

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(sa.LIB_PATH), "sol_attn_example")


@pytest.mark.parametrize("n", [4096, 1000])
def test_c_example_runs(n):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), "C example not built: run python -m block_sparse_attention_14_amd.build"
    print(f"C example N={n}", flush=True)
    r = subprocess.run([EXE, str(n)], text=True, capture_output=True, timeout=100)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "tau=8: kept" in r.stdout and "tau=inf: max abs error" in r.stdout
