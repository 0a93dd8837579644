"""Shared helpers for the parity tests: oracle parameters, the near-tie rule
for Top-tau masks, and sampled output checks."""
from __future__ import annotations

import numpy as np
import torch

from oracle import rra_oracle as orc

# Near-tie tolerance for masks (a cumulative prefix within this of tau, or two
# masses at the cut within this relative gap, may legitimately be cut either
# way by float32 vs float64 arithmetic).
TIE_TOL = 1e-4
SCORE_ATOL = 1e-5  # block scores, float32 GPU vs float64 oracle
OUT_ATOL = 1e-2  # attention outputs, bf16 inputs with float32 accumulation


def out_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Max error of a bf16 output beyond the rounding of the output itself.

    The library returns bf16, so even a perfect kernel differs from the exact
    (float64 oracle) value by up to half a bf16 ulp of that value; with
    unit-variance V that alone exceeds 1e-2 for |out| >= 4.  The tolerance
    bounds what is left: max(|got - ref| - ulp_bf16(ref) / 2)."""
    ref = np.asarray(ref, dtype=np.float64)
    _, ex = np.frexp(np.abs(ref))
    half_ulp = np.ldexp(1.0, np.maximum(ex - 1, -126) - 8)
    return float(np.max(np.abs(got - ref) - half_ulp))


def oracle_params(w, tau=None, stride=None, protect_last=True, rr_mode="head", rr_layer=0,
                  rr_fixed=0) -> orc.Params:
    t = w.tau if tau is None else tau
    return orc.Params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim,
                      w.stride if stride is None else stride, w.block,
                      float(np.float32(t)), protect_last, rr_mode=rr_mode, rr_layer=rr_layer,
                      rr_fixed=rr_fixed)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy()


def _order(vals):
    n = vals.size
    return np.lexsort((np.arange(n), -vals))


def compare_masks(gpu_mask, gpu_cnt, gpu_idx, m_oracle, prm: orc.Params, heads=None):
    """Compare GPU selections with the oracle's, row by row.

    Rows equal to the oracle pass.  A differing row must be a near-tie (an
    oracle prefix within TIE_TOL of tau, or masses at the cut within TIE_TOL
    relative) and must still be a valid Top-tau selection under the oracle's
    masses.  Returns (rows_checked, near_tie_rows, bad_rows)."""
    B, H, nb, _ = gpu_mask.shape
    heads = range(H) if heads is None else heads
    checked = near = 0
    bad = []
    for b in range(B):
        for h in heads:
            for i in range(nb):
                checked += 1
                n = i + 1 if prm.causal else nb  # candidate key blocks
                gsel = np.nonzero(gpu_mask[b, h, i, :n])[0]
                assert np.all(gpu_mask[b, h, i, n:] == 0), "mask above the diagonal"
                assert gpu_cnt[b, h, i] == gsel.size, "count does not match the mask"
                assert np.array_equal(gpu_idx[b, h, i, :gsel.size], gsel), "index list is not the ascending mask"
                osel = orc.top_tau_row(m_oracle[b, h, i], i, prm.tau, prm.protect_last and i == nb - 1,
                                       prm.causal)
                if np.array_equal(gsel, osel):
                    continue
                vals = m_oracle[b, h, i, :n]
                T = vals.sum()
                if not T > 0:
                    bad.append((b, h, i, "row without an estimate must keep every candidate"))
                    continue
                order = _order(vals)
                csum = np.cumsum(vals[order]) / T
                ks = osel.size
                prefix_tie = np.any(np.abs(csum - prm.tau) < TIE_TOL)
                mass_tie = ks < n and abs(vals[order[ks - 1]] - vals[order[ks]]) < TIE_TOL * vals[order[ks - 1]]
                if not (prefix_tie or mass_tie):
                    bad.append((b, h, i, "differs without a near tie"))
                    continue
                near += 1
                gm = vals[gsel].sum()
                unsel = np.setdiff1d(np.arange(n), gsel)
                ok = gm >= (prm.tau - TIE_TOL) * T
                ok &= abs(gsel.size - ks) <= 1
                if unsel.size:
                    ok &= vals[gsel].min() >= vals[unsel].max() * (1 - TIE_TOL) - 1e-12
                ok &= gm - vals[gsel].min() < (prm.tau + TIE_TOL) * T
                if not ok:
                    bad.append((b, h, i, "near tie but not a valid Top-tau set"))
    return checked, near, bad


def check_output_rows(out_gpu, q, k, v, mask, prm: orc.Params, rows):
    """Max-abs error of GPU output rows against the oracle on the given mask."""
    worst = 0.0
    for (b, h, i) in rows:
        ref = orc.attention_rows(q, k, v, mask, prm, b, h, i)
        got = to_f64(out_gpu[b, h, i * prm.block:(i + 1) * prm.block])
        worst = max(worst, out_err(got, ref))
    return worst


REL_FLOOR = 1e-2  # relative errors are taken over output elements with |exact| >= this


def output_errors(got: np.ndarray, ref: np.ndarray) -> dict:
    """Error figures of bf16 outputs against the exact values: the bar's error
    (beyond the output's own half-ulp rounding), the raw max-abs, and the max
    relative error over elements whose exact value is at least REL_FLOOR."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = np.abs(got - ref)
    big = np.abs(ref) >= REL_FLOOR
    return {"err": out_err(got, ref), "max_abs": float(diff.max()),
            "max_rel": float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0}


def merge_errors(a: dict | None, b: dict) -> dict:
    return dict(b) if a is None else {k: max(a[k], b[k]) for k in b}


def seeded_rows(seed: int, batch: int, heads: int, nb: int, n: int = 64):
    """n distinct seeded (b, h, query block) rows, always including the first
    and the last query block."""
    rng = np.random.default_rng(seed)
    rows = {(0, 0, nb - 1), (batch - 1, heads - 1, 0)}
    while len(rows) < min(n, batch * heads * nb):
        rows.add((int(rng.integers(batch)), int(rng.integers(heads)), int(rng.integers(nb))))
    return sorted(rows)


def check_rows_by_head(out, q, k, v, mask, prm: orc.Params, rows) -> dict:
    """Output rows against the oracle on the given mask, converting one head of
    the CPU bf16 tensors q, k, v (torch) to float64 at a time, so that
    full-size workloads need no float64 copy of the whole layer.  Returns the
    merged output_errors of all rows."""
    one = orc.Params(1, 1, 1, prm.seq_len, prm.head_dim, prm.stride, prm.block, prm.tau, prm.protect_last,
                     prm.sm_scale, causal=prm.causal)
    kv_cache = {}
    res = None
    by_head = {}
    for (b, h, i) in rows:
        by_head.setdefault((b, h), []).append(i)
    for (b, h), blocks in sorted(by_head.items()):
        g = h // prm.group
        if (b, g) not in kv_cache:
            kv_cache.clear()
            kv_cache[(b, g)] = (to_f64(k[b:b + 1, g:g + 1]), to_f64(v[b:b + 1, g:g + 1]))
        kh, vh = kv_cache[(b, g)]
        qh = to_f64(q[b:b + 1, h:h + 1])
        mh = np.asarray(mask[b:b + 1, h:h + 1])
        for i in blocks:
            ref = orc.attention_rows(qh, kh, vh, mh, one, 0, 0, i)
            got = to_f64(out[b, h, i * prm.block:i * prm.block + ref.shape[0]])
            res = merge_errors(res, output_errors(got, ref))
    return res
