"""Exact block masses (rra_block_mass) and the exact Top-tau selection made
from them, against the oracle (needs gfx950).

Bars: masses within 1e-5 absolute of the float64 oracle (every cell at small
sizes, sampled rows at 32K); the exact selection made by rra_top_tau from the
GPU masses equals the oracle's selection from its own masses except near-tie
rows, which must be valid Top-tau sets.
"""
import os
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sample_amd as rra
from dynamic_block_sparse_sample_amd import workloads as wl
from dynamic_block_sparse_sample_amd.selection import selection_accuracy
from oracle import rra_oracle as orc

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from helpers import SCORE_ATOL, compare_masks, oracle_params, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def say(*a):
    print(*a, flush=True)


# (name, B, H, Hkv, L, d, S, Bk, tau): every kernel template, G in {1, 2, 4, 7}
SHAPES = [
    ("d128_bk128", 1, 8, 2, 2048, 128, 16, 128, 0.9),
    ("d128_bk64", 1, 4, 2, 1024, 128, 8, 64, 0.9),
    ("d64_bk128_b2", 2, 4, 1, 1024, 64, 8, 128, 0.8),
    ("d64_bk64", 1, 4, 4, 1024, 64, 8, 64, 0.95),
    ("g7", 1, 7, 1, 1152, 128, 16, 128, 0.9),
    ("single_block", 1, 2, 1, 128, 128, 16, 128, 0.9),
]


@pytest.mark.parametrize("case", SHAPES, ids=[c[0] for c in SHAPES])
def test_block_mass_and_exact_selection(case):
    name, B, H, Hkv, L, d, S, Bk, tau = case
    say("case", case)
    q, k, _ = wl.make_random(B, H, Hkv, L, d, seed=5, scale=1.5, diag=1.0)
    prm = orc.Params(B, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    mass = rra.block_mass(p, q.cuda(), k.cuda())
    torch.cuda.synchronize()
    ref = orc.exact_block_mass(to_f64(q), to_f64(k), prm)
    err = float(np.max(np.abs(to_f64(mass) - ref)))
    say(f"  mass max-abs {err:.2e}")
    assert err <= SCORE_ATOL
    nb = L // Bk
    up = np.triu_indices(nb, k=1)
    assert np.all(to_f64(mass)[..., up[0], up[1]] == 0)
    mask, idx, cnt = rra.top_tau(p, mass)
    torch.cuda.synchronize()
    checked, near, bad = compare_masks(mask.cpu().numpy(), cnt.cpu().numpy(), idx.cpu().numpy(), ref, prm)
    say(f"  exact-selection rows {checked}, near-tie rows {near}")
    assert not bad, bad[:5]


def test_block_mass_llama_32k_sampled_rows_and_accuracy():
    w = wl.WORKLOADS["llama_32k"]
    q, k, _ = wl.make_inputs(w)
    qd, kd = q.cuda(), k.cuda()
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, 16, w.block, 0.9)
    prm = oracle_params(w, tau=0.9, stride=16)
    mass = rra.block_mass(p, qd, kd)
    torch.cuda.synchronize()
    rows_sum = mass.double().sum(-1)
    assert torch.allclose(rows_sum, torch.ones_like(rows_sum), atol=1e-4)
    mn = to_f64(mass)
    worst = 0.0
    for h, i in [(0, 255), (1, 100), (13, 17), (31, 0), (22, 254)]:
        ref = orc.exact_block_mass_row(to_f64(q), to_f64(k), prm, 0, h, i)
        worst = max(worst, float(np.max(np.abs(mn[0, h, i] - ref))))
    say(f"llama_32k sampled mass rows: max-abs {worst:.2e}")
    assert worst <= SCORE_ATOL
    # exact vs estimated selection: every metric in range; the exact set keeps >= tau of the mass
    ex_mask, _, _ = rra.top_tau(p, mass)
    est = rra.estimate(p, qd, kd)
    torch.cuda.synchronize()
    r = selection_accuracy(est.mask, ex_mask, mass, 0.9)
    say("llama_32k S=16 tau=0.9 accuracy:", {kk: (round(v, 4) if isinstance(v, float) else v) for kk, v in r.items()})
    assert 0.0 <= r["precision"] <= 1.0 and 0.0 <= r["recall"] <= 1.0
    kept_exact = (mass.double() * ex_mask.double()).sum(-1)
    assert float(kept_exact.min()) >= 0.9 * float(rows_sum.min()) - 1e-5
