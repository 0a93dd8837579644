"""The whole path from a C program, through the C ABI only (needs gfx950).

tests/c_abi/gpu_path.c (built by __graft_entry__.build() into _build/) takes
device buffers from the HIP runtime, runs rra_estimate, rra_sparse_attn on
both schedules and rra_dense_attn, and checks what holds for any input: at
tau = 1 every causal block kept and sparse bitwise equal to dense; at tau = 0.9
well-formed ascending lists matching the mask, the protected last row whole,
finite outputs, and the two schedules bitwise equal.
"""
import os
import subprocess

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "_build", "rra_c_gpu_path")


def test_c_program_runs_the_path():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(EXE), f"{EXE} is missing: run __graft_entry__.build()"
    print("running", EXE, flush=True)
    run = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(run.stdout, run.stderr, flush=True)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip().splitlines()[-1] == "ok"
