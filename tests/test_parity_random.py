"""Seeded random configurations, every step against the oracle (needs gfx950).

Twenty-four valid problems drawn from fixed seeds mix what the other parity
tests vary one at a time: batch 1-2, grouped-query ratios 1-7, head dims 64
and 128, blocks of 64 and 128 with every stride that divides them (up to 32
strides per block), lengths from 1 to 6000 (mostly ragged), tau from 0.5 to
1, causal or not, last-row protection on or off, the four round-robin
strategies and explicit softmax scales.  Bars as elsewhere: Kagg bit-exact,
block scores and exact block masses within 1e-5, Top-tau on identical scores
bit-exact, estimator masks under the near-tie rule, attention outputs within
1e-2 beyond their own bf16 rounding (sparse on the GPU's own mask, and dense).
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
from helpers import OUT_ATOL, SCORE_ATOL, compare_masks, out_err, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


def _draw_cases(n=16, seed=2026, first=0, lengths=(1, 1601), max_hkv=4):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(first, first + n):
        d = int(rng.choice([64, 128]))
        bk = int(rng.choice([64, 128]))
        strides = [s for s in (2, 4, 8, 16, 32, 64, 128) if bk % s == 0 and bk // s <= 32]
        S = int(rng.choice(strides))
        hkv = int(rng.choice([h for h in (1, 2, 4) if h <= max_hkv]))
        G = int(rng.choice([1, 2, 3, 4, 7]))
        B = int(rng.choice([1, 2]))
        L = int(rng.integers(*lengths))
        tau = float(rng.choice([0.5, 0.8, 0.9, 0.95, 0.99, 1.0]))
        causal = bool(rng.random() < 0.7)
        protect = bool(rng.random() < 0.6)
        mode = str(rng.choice(["head", "layer", "hybrid", "none"]))
        layer = int(rng.integers(0, 40))
        fixed = int(rng.integers(0, S))
        scale = float(rng.choice([0.0, 0.05, 0.2]))
        cases.append((f"r{i:02d}", B, hkv * G, hkv, L, d, S, bk, tau, causal, protect, mode, layer, fixed, scale))
    return cases


# Longer rows (up to 94 blocks of 64: the selection's second register slot;
# 24-47 blocks of 128), fewer heads so the oracle stays fast.
CASES = _draw_cases() + _draw_cases(n=8, seed=4051, first=16, lengths=(3000, 6001), max_hkv=2)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_random_config_all_steps(case):
    name, B, H, Hkv, L, d, S, Bk, tau, causal, protect, mode, layer, fixed, scale = case
    say("case", case)
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=31 + int(name[1:]), scale=1.5, diag=1.0)
    prm = orc.Params(B, H, Hkv, L, d, S, Bk, float(np.float32(tau)), protect, sm_scale=float(np.float32(scale)),
                     rr_mode=mode, rr_layer=layer, rr_fixed=fixed, causal=causal)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau, protect_last=protect, sm_scale=scale, causal=causal,
                        rr_mode=mode, rr_layer=layer, rr_offset=fixed)
    assert p.num_blocks == prm.num_blocks and p.num_strides == prm.num_strides
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)

    kagg = rra.stride_aggregate(p, kd)
    for b in range(B):
        for g in range(Hkv):
            assert np.array_equal(to_f64(kagg[b, g]), orc.aggregate_keys(kn[b, g], S, "bf16"))
    score = rra.block_scores(p, qd, kagg)
    m_or = orc.block_scores(qn, kn, prm)
    err = float(np.max(np.abs(to_f64(score) - m_or)))
    say(f"  block score max-abs {err:.2e}")
    assert err <= SCORE_ATOL

    mask, idx, cnt = rra.top_tau(p, score)
    torch.cuda.synchronize()
    omask, oidx, ocnt = orc.select_blocks(to_f64(score), prm)
    assert np.array_equal(mask.cpu().numpy(), omask)
    assert np.array_equal(cnt.cpu().numpy(), ocnt)

    sel = rra.estimate(p, qd, kd, return_score=True)
    torch.cuda.synchronize()
    assert torch.equal(sel.score, score)
    checked, near, bad = compare_masks(sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(),
                                       m_or, prm)
    say(f"  mask rows {checked}, near-tie rows {near}")
    assert not bad, bad[:5]

    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    dense = rra.dense_attn(p, qd, kd, vd)
    mass = rra.block_mass(p, qd, kd)
    torch.cuda.synchronize()
    e_sp = out_err(to_f64(out), orc.block_sparse_attention(qn, kn, vn, sel.mask.cpu().numpy(), prm))
    e_dn = out_err(to_f64(dense), orc.dense_attention(qn, kn, vn, prm))
    e_ms = float(np.max(np.abs(to_f64(mass) - orc.exact_block_mass(qn, kn, prm))))
    say(f"  sparse {e_sp:.2e}, dense {e_dn:.2e}, exact mass {e_ms:.2e}")
    assert e_sp <= OUT_ATOL and e_dn <= OUT_ATOL and e_ms <= SCORE_ATOL
