"""Selection-accuracy metrics on a hand-worked example (CPU)."""
import pytest
import torch

from dynamic_block_sparse_sample_amd.selection import selection_accuracy


def test_hand_worked_counts_and_mass():
    exact = torch.tensor([[1, 0, 0], [1, 1, 0], [0, 1, 1]], dtype=torch.uint8)[None, None]
    est = torch.tensor([[1, 0, 0], [0, 1, 0], [1, 1, 1]], dtype=torch.uint8)[None, None]
    mass = torch.tensor([[1.0, 0, 0], [0.3, 0.7, 0], [0.05, 0.45, 0.5]])[None, None]
    r = selection_accuracy(est, exact, mass, tau=0.9)
    assert (r["tp"], r["fp"], r["fn"]) == (4, 1, 1)
    assert r["precision"] == pytest.approx(0.8) and r["recall"] == pytest.approx(0.8)
    assert r["f1"] == pytest.approx(0.8)
    assert r["density_estimated"] == pytest.approx(5 / 6) and r["density_exact"] == pytest.approx(5 / 6)
    assert r["mass_kept_mean"] == pytest.approx((1.0 + 0.7 + 1.0) / 3)
    assert r["mass_kept_min"] == pytest.approx(0.7)
    assert r["rows_below_tau"] == pytest.approx(1 / 3)
    assert r["exact_mass_kept_mean"] == pytest.approx((1.0 + 1.0 + 0.95) / 3)


def test_identical_selections_are_perfect():
    g = torch.Generator().manual_seed(0)
    m = torch.tril(torch.randint(0, 2, (2, 3, 8, 8), generator=g)).to(torch.uint8)
    m[..., 0] = 1
    mass = torch.tril(torch.rand(2, 3, 8, 8, generator=g))
    mass = mass / mass.sum(-1, keepdim=True)
    r = selection_accuracy(m, m, mass, tau=0.5)
    assert r["precision"] == 1.0 and r["recall"] == 1.0 and r["f1"] == 1.0
    assert r["mass_kept_mean"] == pytest.approx(r["exact_mass_kept_mean"])
