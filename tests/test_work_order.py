"""The attention kernel's work order, checked on the CPU.

`csrc/kernels/fa_order.h` holds the item -> (KV row, head, query block)
mapping and the phase sizing that `flash_attn.hip` uses, as constexpr C++.
`tests/c_abi/work_order.cpp` includes the same header, built here with the
host compiler: for the workload shapes and a grid of batch sizes, group
counts, GQA ratios and ragged lengths, under both phase budgets, every row is
an item exactly once and the XCD / phase / head-adjacency structure holds.  It
also confirms the checker catches the one mistake this order once had (a
phase size that does not divide the group count).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_work_order_is_a_bijection(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    src = os.path.join(ROOT, "tests", "c_abi", "work_order.cpp")
    inc = os.path.join(ROOT, "dynamic_block_sparse_sample_amd", "csrc", "kernels")
    exe = str(tmp_path / "work_order")
    subprocess.run([gxx, "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror", f"-I{inc}", "-o", exe, src],
                   check=True, capture_output=True, text=True, timeout=120)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-2000:]
    assert run.stdout.strip().endswith("ok")
