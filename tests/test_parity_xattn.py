"""XAttention's antidiagonal block scores (rra_xattn_block_scores, the
comparison estimator) against the oracle (needs gfx950).

Bars: scores within 1e-5 of the float64 oracle; the selection rra_top_tau
makes from them equals the oracle's under the near-tie rule.
"""
import os
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sample_amd as rra
from dynamic_block_sparse_sample_amd import workloads as wl
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


# (name, B, H, Hkv, L, d, S, Bk, tau): every template (R, S/4) for d 64 and 128, G in {1, 2, 4, 7}
CASES = [
    ("d128_bk128_s16", 1, 8, 2, 2048, 128, 16, 128, 0.9),
    ("d128_bk128_s8", 1, 4, 2, 2048, 128, 8, 128, 0.9),
    ("d128_bk128_s4_g1", 1, 2, 2, 1024, 128, 4, 128, 0.95),
    ("d64_bk64_s8_b2", 2, 4, 1, 1024, 64, 8, 64, 0.8),
    ("d64_bk64_s4", 1, 4, 4, 1024, 64, 4, 64, 0.9),
    ("d64_bk128_s16_g7", 1, 7, 1, 1024, 64, 16, 128, 0.9),
    ("single_block", 1, 4, 1, 128, 128, 16, 128, 0.9),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_xattn_scores_and_selection(case):
    name, B, H, Hkv, L, d, S, Bk, tau = case
    say("case", case)
    q, k, _ = wl.make_random(B, H, Hkv, L, d, seed=9, scale=1.5, diag=1.0)
    prm = orc.Params(B, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    score = rra.xattn_block_scores(p, q.cuda(), k.cuda())
    mask, idx, cnt = rra.top_tau(p, score)
    torch.cuda.synchronize()
    ref = orc.xattn_block_scores(to_f64(q), to_f64(k), prm)
    err = float(np.max(np.abs(to_f64(score) - ref)))
    checked, near, bad = compare_masks(mask.cpu().numpy(), cnt.cpu().numpy(), idx.cpu().numpy(), ref, prm)
    say(f"  score max-abs {err:.2e}, mask rows {checked}, near-tie rows {near}")
    assert err <= SCORE_ATOL
    assert not bad, bad[:5]


def test_xattn_llama_32k_sampled_heads():
    w = wl.WORKLOADS["llama_32k"]
    q, k, _ = wl.make_inputs(w)
    for S in (16, 8):
        p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, 0.9)
        prm = oracle_params(w, tau=0.9, stride=S)
        score = rra.xattn_block_scores(p, q.cuda(), k.cuda())
        torch.cuda.synchronize()
        rows = score.double().sum(-1)
        assert torch.allclose(rows, torch.ones_like(rows), atol=1e-4)
        for h in (0, 13):
            one = orc.Params(1, 1, 1, w.seq_len, w.head_dim, S, w.block, prm.tau, True)
            ref = orc.xattn_block_scores(to_f64(q[:, h:h + 1]), to_f64(k[:, h // 4:h // 4 + 1]), one)
            err = float(np.max(np.abs(to_f64(score[0, h]) - ref[0, 0])))
            say(f"llama_32k S={S} head {h}: xattn score max-abs {err:.2e}")
            assert err <= SCORE_ATOL
