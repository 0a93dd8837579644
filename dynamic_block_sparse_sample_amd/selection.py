"""Scoring an estimated block selection against the exact one.

Reporting only (torch operations on the library's outputs): the exact
selection is Top-tau applied to the exact block masses of full causal
attention (rra_block_mass, then rra_top_tau), and the estimated one is the
round-robin estimator's mask (rra_estimate).  Counts run over the causal
cells J <= I of every (batch, head, query-block) row, the protected last row
included (both selections keep it whole).
"""
from __future__ import annotations

import torch


def selection_accuracy(est_mask: torch.Tensor, exact_mask: torch.Tensor, exact_mass: torch.Tensor,
                       tau: float) -> dict:
    """Precision, recall and F1 of est_mask against exact_mask, and the exact
    attention mass each keeps per row (rows of exact_mass sum to 1).

    est_mask, exact_mask: [Bz, H, Nb, Nb] uint8/bool, zero above the diagonal;
    exact_mass: [Bz, H, Nb, Nb] float.
    """
    est = est_mask.bool()
    ex = exact_mask.bool()
    nb = est.shape[-1]
    rows = est.shape[0] * est.shape[1] * nb
    causal = rows * (nb + 1) / 2 if rows else 0
    tp = int((est & ex).sum())
    fp = int((est & ~ex).sum())
    fn = int((~est & ex).sum())
    precision = tp / (tp + fp) if tp + fp else 1.0
    recall = tp / (tp + fn) if tp + fn else 1.0
    f1 = 2 * precision * recall / (precision + recall) if precision + recall else 0.0
    mass = exact_mass.double()
    kept = (mass * est.double()).sum(-1).flatten()
    kept_exact = (mass * ex.double()).sum(-1).flatten()
    return {
        "precision": precision,
        "recall": recall,
        "f1": f1,
        "tp": tp, "fp": fp, "fn": fn,
        "density_estimated": int(est.sum()) / causal if causal else 0.0,
        "density_exact": int(ex.sum()) / causal if causal else 0.0,
        "mass_kept_mean": float(kept.mean()) if rows else 1.0,
        "mass_kept_p01": float(torch.quantile(kept.float(), 0.01)) if rows else 1.0,
        "mass_kept_min": float(kept.min()) if rows else 1.0,
        "rows_below_tau": float((kept < tau - 1e-6).double().mean()) if rows else 0.0,
        "exact_mass_kept_mean": float(kept_exact.mean()) if rows else 1.0,
    }
