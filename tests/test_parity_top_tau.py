"""Top-tau selection on given score rows against the oracle (needs gfx950).

The scores are synthetic and handed to rra_top_tau directly, so both sides
select on identical float32 values.  Rows whose sums are exact in float64
(dyadic values, equal values, one-hot rows, all-zero rows) must match the
oracle bit for bit, ties resolved by the lowest J; rows of general values
(a wide dynamic range, denormals) follow the near-tie rule.  Sizes straddle
the 64-block register slots (63, 64, 65, 1024, 1025) up to 4096 blocks,
causal (entries above the diagonal hold junk that must never be read) and
not, with and without last-row protection, tau from 0.5 to 1.
"""
import os
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sample_amd as rra
from oracle import rra_oracle as orc

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from helpers import compare_masks  # noqa: E402

pytestmark = pytest.mark.gpu

EXACT_KINDS = ("dyadic", "constant", "onehot", "zeros_and_ties")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def say(*a):
    print(*a, flush=True)


def make_scores(kind: str, heads: int, nb: int, causal: bool, seed: int) -> np.ndarray:
    """Score rows [1, heads, nb, nb] float32 of the given structure (seeded)."""
    rng = np.random.default_rng(seed)
    s = np.zeros((1, heads, nb, nb), dtype=np.float32)
    cols = np.arange(nb)
    for h in range(heads):
        u = rng.random((nb, nb))
        if kind == "dyadic":  # values k/16, k = 0..4: many exact ties and zeros
            rows = np.floor(u * 5) / 16
        elif kind == "constant":  # one value per row: every candidate tied
            rows = np.repeat(rng.integers(1, 9, size=(nb, 1)) / 64.0, nb, axis=1)
        elif kind == "onehot":
            rows = np.zeros((nb, nb))
            hot = (u[:, 0] * (np.arange(nb) + 1 if causal else nb)).astype(np.int64)
            rows[np.arange(nb), hot] = 1.0
        elif kind == "zeros_and_ties":  # mostly zero rows, some rows of two tied values
            rows = np.where(u < 0.9, 0.0, 0.25)
            rows[::3] = 0.0  # whole rows without an estimate: keep every candidate
        elif kind == "wide":  # masses over ~20 orders of magnitude, normalised
            rows = u ** 40
            rows /= rows.sum(axis=1, keepdims=True)
        elif kind == "denormal":  # float32 denormals and small normals
            rows = np.floor(u * 2 ** 12) * 2.0 ** -140
        else:
            raise ValueError(kind)
        rows = rows.astype(np.float32)
        if causal:  # junk above the diagonal: never a candidate
            rows[cols[None, :] > cols[:, None]] = 3.0
        s[0, h] = rows
    return s


def run_top_tau(scores: np.ndarray, tau: float, protect: bool, causal: bool):
    _, H, nb, _ = scores.shape
    blk = 64
    p = rra.make_params(1, H, H, nb * blk, 64, 8, blk, tau, protect_last=protect, causal=causal)
    prm = orc.Params(1, H, H, nb * blk, 64, 8, blk, float(np.float32(tau)), protect, causal=causal)
    sc = torch.from_numpy(scores).cuda()
    mask = torch.full((1, H, nb, nb), 9, dtype=torch.uint8, device="cuda")
    idx = torch.full((1, H, nb, nb), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((1, H, nb), -7, dtype=torch.int32, device="cuda")
    rra.top_tau(p, sc, mask=mask, idx=idx, cnt=cnt)
    torch.cuda.synchronize()
    return mask.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy(), prm


def check_exact(mask, idx, cnt, scores, prm, rows=None):
    """Every (listed) row equals the oracle's selection; mask, idx and cnt agree."""
    _, H, nb, _ = scores.shape
    rows = [(h, i) for h in range(H) for i in range(nb)] if rows is None else rows
    for h, i in rows:
        n = i + 1 if prm.causal else nb
        want = orc.top_tau_row(scores[0, h, i].astype(np.float64), i, prm.tau,
                               prm.protect_last and i == nb - 1, prm.causal)
        got = np.nonzero(mask[0, h, i])[0]
        assert np.array_equal(got, want), (h, i, got[:12], want[:12])
        assert cnt[0, h, i] == want.size
        assert np.array_equal(idx[0, h, i, :want.size], want)
        assert np.all(mask[0, h, i, n:] == 0)


SIZES = [(1, True), (2, True), (63, True), (64, False), (65, True), (129, False), (700, True)]


@pytest.mark.parametrize("kind", EXACT_KINDS)
@pytest.mark.parametrize("nb,causal", SIZES, ids=[f"nb{n}_{'c' if c else 'nc'}" for n, c in SIZES])
def test_exact_rows(kind, nb, causal):
    for tau, protect in ((0.9, True), (0.5, False), (0.999, False)):
        scores = make_scores(kind, 2, nb, causal, seed=nb * 7 + len(kind))
        mask, idx, cnt, prm = run_top_tau(scores, tau, protect, causal)
        check_exact(mask, idx, cnt, scores, prm)


@pytest.mark.parametrize("kind", ("wide", "denormal"))
@pytest.mark.parametrize("nb,causal", [(65, True), (700, False), (1025, True)])
def test_general_rows_near_tie_rule(kind, nb, causal):
    scores = make_scores(kind, 2, nb, causal, seed=nb + 3)
    mask, idx, cnt, prm = run_top_tau(scores, 0.9, True, causal)
    m = scores.astype(np.float64)
    checked, near, bad = compare_masks(mask, cnt, idx, m, prm)
    say(kind, nb, causal, "rows", checked, "near ties", near)
    assert not bad, bad[:5]
    assert near <= max(1, checked // 1000)


def test_tau_one_keeps_every_candidate():
    scores = make_scores("wide", 2, 300, True, seed=5)
    mask, idx, cnt, prm = run_top_tau(scores, 1.0, False, True)
    assert np.array_equal(cnt[0], np.tile(np.arange(1, 301), (2, 1)))
    check_exact(mask, idx, cnt, scores, prm)


@pytest.mark.parametrize("causal", [True, False])
def test_slot_boundaries_and_4096_blocks(causal):
    """Rows of 1024 and 1025 candidates (16 and 64 register slots) in full;
    4096 blocks on sampled rows spread over every slot class."""
    scores = make_scores("dyadic", 1, 1025, causal, seed=11)
    mask, idx, cnt, prm = run_top_tau(scores, 0.8, False, causal)
    check_exact(mask, idx, cnt, scores, prm)
    scores = make_scores("dyadic", 1, 4096, causal, seed=12)
    mask, idx, cnt, prm = run_top_tau(scores, 0.9, True, causal)
    rows = [(0, i) for i in (0, 1, 62, 63, 64, 127, 128, 255, 256, 511, 512, 1023, 1024, 2047, 2048, 3000,
                             4094, 4095)]
    rows += [(0, int(i)) for i in np.random.default_rng(3).integers(0, 4096, 40)]
    check_exact(mask, idx, cnt, scores, prm, rows)
