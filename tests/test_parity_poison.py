"""Every output and workspace byte the path reads is one it wrote (needs gfx950).

The whole path runs twice on the same inputs: once on zero-filled buffers and
once with every buffer it is handed (estimator workspace holding Kagg and the
block scores, the score, mask, index and count outputs, the attention
schedule workspace and the attention outputs) filled with NaN / junk bytes.
A kernel that read a byte it had not written (a stride, block row or output
row left out, say at a ragged end or above the causal diagonal) would carry
the poison into the results; they must be bitwise those of the clean run
(index lists compared up to their counts, the rest being unspecified).
"""
import pytest
import torch

import dynamic_block_sparse_sample_amd as rra
from dynamic_block_sparse_sample_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


# (name, B, H, Hkv, L, d, S, Bk, tau, causal, protect)
CASES = [
    ("ragged_causal", 1, 8, 2, 3000 + 37, 128, 16, 128, 0.9, True, True),
    ("ragged_noncausal", 2, 4, 1, 2000 + 5, 128, 8, 128, 0.8, False, False),
    ("bk64_d64_ragged", 1, 6, 3, 1500 + 11, 64, 4, 64, 0.95, True, False),
    ("tiny_partial_stride", 1, 4, 4, 100, 64, 8, 64, 0.9, True, True),
    ("many_rows_dynamic", 1, 32, 8, 8192, 128, 16, 128, 0.9, True, True),  # rows > resident workgroups
]


def run_path(p, qd, kd, vd, fill):
    """estimate (scores kept) + sparse + dense attention on buffers pre-filled by `fill`."""
    B, H, L, d = qd.shape
    nb = p.num_blocks
    est_ws = rra.alloc_workspace(p)
    attn_ws = torch.empty(rra.attn_workspace_size(p), dtype=torch.uint8, device="cuda")
    sel = rra.Selection(torch.empty((B, H, nb, nb), dtype=torch.uint8, device="cuda"),
                        torch.empty((B, H, nb, nb), dtype=torch.int32, device="cuda"),
                        torch.empty((B, H, nb), dtype=torch.int32, device="cuda"),
                        torch.empty((B, H, nb, nb), dtype=torch.float32, device="cuda"))
    out = torch.empty_like(qd)
    dense = torch.empty_like(qd)
    for t in (est_ws, attn_ws, sel.mask, sel.idx, sel.cnt, sel.score, out, dense):
        fill(t)
    rra.estimate(p, qd, kd, workspace=est_ws, out=sel)
    rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out, workspace=attn_ws)
    rra.dense_attn(p, qd, kd, vd, out=dense, workspace=attn_ws)
    # the estimator's own score matrix in its workspace, via a second call without `score`
    sel2 = rra.Selection(torch.empty_like(sel.mask), torch.empty_like(sel.idx), torch.empty_like(sel.cnt), None)
    for t in (sel2.mask, sel2.idx, sel2.cnt):
        fill(t)
    fill(est_ws)
    rra.estimate(p, qd, kd, workspace=est_ws, out=sel2)
    torch.cuda.synchronize()
    return sel, sel2, out, dense


def zero(t):
    t.zero_()


def poison(t):
    if t.dtype in (torch.float32, torch.bfloat16):
        t.fill_(float("nan"))
    elif t.dtype == torch.uint8:
        t.fill_(0xFF)  # NaN in every float view of the workspaces
    else:
        t.fill_(-123456)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_poisoned_buffers_change_nothing(case):
    name, B, H, Hkv, L, d, S, Bk, tau, causal, protect = case
    print("case", case, flush=True)
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=17, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau, protect_last=protect, causal=causal)
    nb = p.num_blocks
    clean = run_path(p, qd, kd, vd, zero)
    dirty = run_path(p, qd, kd, vd, poison)
    valid = torch.arange(nb, device="cuda").view(1, 1, 1, nb) < clean[0].cnt.unsqueeze(-1)
    for a, b in ((clean[0], dirty[0]), (clean[1], dirty[1])):
        assert torch.equal(a.mask, b.mask)
        assert torch.equal(a.cnt, b.cnt)
        assert torch.equal(torch.where(valid, a.idx, 0), torch.where(valid, b.idx, 0))
    assert torch.equal(clean[0].score, dirty[0].score)
    assert torch.isfinite(dirty[0].score).all()
    assert torch.equal(clean[2], dirty[2]) and torch.equal(clean[3], dirty[3])
    assert torch.isfinite(dirty[2].float()).all() and torch.isfinite(dirty[3].float()).all()
    assert torch.equal(clean[0].mask, clean[1].mask)  # scores in the workspace select the same blocks
