"""Rows with logits far above their first key sub-tile's (needs gfx950).

The fast pass fixes each row's reference max from its first key sub-tile; a
row whose later logits lie far above it (probabilities past 2^64, or past the
float32 range) makes the whole item run again with the exact running max.
These inputs plant such rows: queries whose first sub-tile holds ordinary
keys and whose later keys include one aligned with the query, with logits
about 100 and about 1000 (base 2) above the rest.  Every output row, the
planted ones included, must match the float64 oracle, on dense attention,
block-sparse attention (an explicit list that skips blocks), and both
schedules (bitwise equal to each other).
"""
import os
import sys

import numpy as np
import pytest
import torch

import dynamic_block_sparse_sample_amd as rra
from oracle import rra_oracle as orc

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from helpers import OUT_ATOL, out_err, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def _inputs(seed, H, Hkv, L, d):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(1, H, L, d, generator=g)
    k = torch.randn(1, Hkv, L, d, generator=g)
    v = torch.randn(1, Hkv, L, d, generator=g)
    # head 0: query 300 (block 2) against key 200 (block 1): q.k = 8 * 0.75 * d
    # (~100 in base-2 logits at d = 128), query 420 (block 3) against key 290
    # (block 2): q.k = 8 * 8 * d (~1000, past the float32 range of 2^x)
    q[0, 0, 300] = 8.0
    k[0, 0, 200] = 0.75
    q[0, 0, 420] = 8.0
    k[0, 0, 290] = 8.0
    return (t.to(torch.bfloat16) for t in (q, k, v))


@pytest.mark.parametrize("d,Bk", [(128, 128), (128, 64), (64, 128)])
def test_rows_past_the_fast_range_are_exact(d, Bk):
    H, Hkv, L, S = 4, 2, 512, 16
    q, k, v = _inputs(7, H, Hkv, L, d)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(1, H, Hkv, L, d, S, Bk, 0.9)
    prm = orc.Params(1, H, Hkv, L, d, S, Bk, float(np.float32(0.9)), True)
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)
    nb = p.num_blocks
    # an explicit list that skips block 0 for every other row (keeps the planted keys' blocks)
    mask = np.tril(np.ones((nb, nb), dtype=np.uint8))
    mask[1::2, 0] = 0
    mask = np.broadcast_to(mask, (1, H, nb, nb)).copy()
    idx = np.zeros((1, H, nb, nb), dtype=np.int32)
    cnt = mask.sum(-1).astype(np.int32)
    for h in range(H):
        for i in range(nb):
            sel = np.nonzero(mask[0, h, i])[0]
            idx[0, h, i, :sel.size] = sel
    idx_d, cnt_d = torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda()
    dense = rra.dense_attn(p, qd, kd, vd)
    dense_static = rra.dense_attn(p, qd, kd, vd, schedule="static")
    sparse = rra.sparse_attn(p, qd, kd, vd, idx_d, cnt_d)
    sparse_static = rra.sparse_attn(p, qd, kd, vd, idx_d, cnt_d, schedule="static")
    torch.cuda.synchronize()
    assert torch.equal(dense, dense_static) and torch.equal(sparse, sparse_static)
    for got, ref in ((dense, orc.dense_attention(qn, kn, vn, prm)),
                     (sparse, orc.block_sparse_attention(qn, kn, vn, mask, prm))):
        g64 = to_f64(got)
        assert np.all(np.isfinite(g64))
        err = out_err(g64, ref)
        print(f"d={d} Bk={Bk}: err {err:.2e}, planted rows "
              f"{np.max(np.abs(g64[0, 0, 300] - ref[0, 0, 300])):.2e} {np.max(np.abs(g64[0, 0, 420] - ref[0, 0, 420])):.2e}",
              flush=True)
        assert err <= OUT_ATOL
        # the planted rows attend (almost) only to their aligned key
        assert np.max(np.abs(ref[0, 0, 420] - vn[0, 0, 290])) < 1e-6


@pytest.mark.parametrize("d,S,Bk", [(128, 16, 128), (64, 8, 64)])
def test_block_scores_rows_past_the_fast_range(d, S, Bk):
    """Stride scores far above the first tile of their row reach the
    estimator's softmax.  Head 0 samples offset 0.  Its query at token 100 S
    (channels [0, d/2) = 8) is aligned with the keys of stride 50 (the same
    channels = 8): a base-2 logit about 520 above the rest (370 at d = 64),
    past the float32 range, so the denominator overflows and pass 1 runs
    again with the exact max.  Its query at token 120 S (channels [d/2, d) = 8)
    is aligned with the keys of stride 70 (the same channels = 0.92): about 60
    above the rest (42 at d = 64), which keeps the denominator finite but puts
    probabilities far above 1 against the first tile's reference.  Every key of a planted stride
    is equal, so its mean is exact.  Block scores within 1e-5 of the oracle
    and masks under the near-tie rule."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from helpers import SCORE_ATOL, compare_masks  # noqa: E402
    H, Hkv, L = 4, 2, 2048
    g = torch.Generator().manual_seed(11)
    q = torch.randn(1, H, L, d, generator=g)
    k = torch.randn(1, Hkv, L, d, generator=g)
    h2 = d // 2
    q[0, 0, 100 * S, :h2] = 8.0
    q[0, 0, 100 * S, h2:] = 0.0
    k[0, 0, 50 * S:51 * S, :h2] = 8.0
    q[0, 0, 120 * S, :h2] = 0.0
    q[0, 0, 120 * S, h2:] = 8.0
    k[0, 0, 70 * S:71 * S, h2:] = 0.92
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    p = rra.make_params(1, H, Hkv, L, d, S, Bk, 0.9)
    prm = orc.Params(1, H, Hkv, L, d, S, Bk, float(np.float32(0.9)), True)
    sel = rra.estimate(p, q.cuda(), k.cuda(), return_score=True)
    torch.cuda.synchronize()
    m_or = orc.block_scores(to_f64(q), to_f64(k), prm)
    got = to_f64(sel.score)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - m_or)))
    for tok, stride in ((100 * S, 50), (120 * S, 70)):
        row, col = tok // Bk, (stride * S) // Bk
        print(f"d={d} S={S}: planted row {row} mass on block {col}: GPU {got[0, 0, row, col]:.4f}, "
              f"oracle {m_or[0, 0, row, col]:.4f}", flush=True)
        assert m_or[0, 0, row, col] > 0.1  # the planted stride dominates its query's softmax
    print(f"d={d} S={S}: score err {err:.2e}", flush=True)
    assert err <= SCORE_ATOL
    checked, near, bad = compare_masks(sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(),
                                       m_or, prm)
    assert not bad, bad[:3]
