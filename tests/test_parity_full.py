"""GPU vs oracle at the workloads' full sizes (needs gfx950).

Masks: every head's every row is compared with the oracle's own masses under
the near-tie rule, at 32K (all nine S x tau points), 64K (video) and 128K (the
benchmarked workload, in the benchmark's launch configuration; one test per KV
group so that each stays within a couple of minutes of CPU work).  Outputs: 64
seeded (head, query block) rows per configuration point, computed by the
oracle one by one on the GPU's own mask.  Properties that hold at any size
(score rows sum to 1, masks agree with their index lists and counts, the
protected last row is full) are checked on every row.  Near-tie counts and the
output errors (the bar's, the raw max-abs, the max relative) are printed per
configuration.
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
from helpers import (OUT_ATOL, SCORE_ATOL, check_rows_by_head, compare_masks, oracle_params,  # noqa: E402
                     seeded_rows, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def say(*a):
    print(*a, flush=True)


def _head_scores(q, kagg, prm, h):
    """Oracle block scores of one query head from its KV group's aggregated keys: [Nb, Nb]."""
    s = orc.stride_scores(to_f64(q[0, h]), kagg, prm.stride, h, prm.scale, prm.rr_mode, prm.rr_layer,
                          prm.rr_fixed, prm.causal)
    return orc.pool_blocks(orc.stride_softmax(s), prm.strides_per_block)


def _check_any_size(sel, p):
    """Properties that hold at any size, on every head and row."""
    nb = p.num_blocks
    score = sel.score
    rows = score.sum(dim=-1)
    assert torch.allclose(rows, torch.ones_like(rows), atol=1e-4), float((rows - 1).abs().max())
    cnt = sel.cnt.long()
    assert torch.equal(sel.mask.long().sum(-1), cnt)
    assert int(cnt.min()) >= 1
    i_idx = torch.arange(nb, device=cnt.device)
    if p.causal:
        assert torch.all(cnt <= i_idx + 1)
        tri = torch.triu(torch.ones(nb, nb, dtype=torch.bool, device=cnt.device), 1)
        assert not torch.any(sel.mask.bool() & tri)
        assert not torch.any(score.masked_select(tri.expand_as(score)) != 0)
    if p.protect_last:
        assert torch.all(cnt[..., -1] == nb)


def _params(w, tau=None, stride=None):
    t = w.tau if tau is None else tau
    s = w.stride if stride is None else stride
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, s, w.block, t)
    return p, oracle_params(w, tau=t, stride=s)


class _Sel:
    """A selection copied to the host: mask, count and index lists as numpy, scores as float64."""

    def __init__(self, sel):
        self.mask = sel.mask.cpu().numpy()
        self.cnt = sel.cnt.cpu().numpy()
        self.idx = sel.idx.cpu().numpy()
        self.score = to_f64(sel.score) if sel.score is not None else None


def _compare_heads(hsel: _Sel, q, k, prm, heads, cache=None):
    """Scores and masks of the given heads against the oracle; returns the near-tie row count."""
    near = 0
    kagg = {}
    for h in heads:
        if cache is not None and h in cache:
            m_h = cache[h]
        else:
            g = h // prm.group
            if g not in kagg:
                kagg = {g: orc.aggregate_keys(to_f64(k[0, g]), prm.stride)}
            m_h = _head_scores(q, kagg[g], prm, h)
            if cache is not None:
                cache[h] = m_h
        err = float(np.max(np.abs(hsel.score[0, h] - m_h)))
        assert err <= SCORE_ATOL, (h, err)
        m_full = np.zeros((1, prm.num_heads) + m_h.shape)
        m_full[0, h] = m_h
        _, n_near, bad = compare_masks(hsel.mask, hsel.cnt, hsel.idx, m_full, prm, heads=[h])
        assert not bad, (h, bad[:3])
        near += n_near
    return near


def _density(cnt, p):
    return float(cnt.sum()) / (p.batch * p.num_heads * p.num_blocks * (p.num_blocks + 1) / 2)


def _report_outputs(label, out, q, k, v, mask, prm, seed):
    rows = seeded_rows(seed, prm.batch, prm.num_heads, prm.num_blocks, 64)
    e = check_rows_by_head(out, q, k, v, mask, prm, rows)
    say(f"{label}: {len(rows)} seeded output rows: err {e['err']:.2e} (bar {OUT_ATOL}), "
        f"raw max-abs {e['max_abs']:.2e}, max-rel {e['max_rel']:.2e}")
    assert e["err"] <= OUT_ATOL, e


# ---------------------------------------------------------------------------
# 32K: every head, all nine S x tau points
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def llama_32k():
    w = wl.WORKLOADS["llama_32k"]
    q, k, v = wl.make_inputs(w)
    return w, q, k, v, q.cuda(), k.cuda(), v.cuda()


@pytest.mark.parametrize("stride", [8, 16, 32])
def test_llama_32k_sweep_every_head(llama_32k, stride):
    """All three taus of one stride (the oracle's block scores are shared),
    every head's mask; 64 seeded output rows on the tau = 0.9 mask."""
    w, q, k, v, qd, kd, vd = llama_32k
    cache = {}
    for tau in (0.8, 0.9, 0.95):
        p, prm = _params(w, tau=tau, stride=stride)
        sel = rra.estimate(p, qd, kd, return_score=True)
        torch.cuda.synchronize()
        _check_any_size(sel, p)
        hsel = _Sel(sel)
        near = _compare_heads(hsel, q, k, prm, range(w.num_heads), cache)
        say(f"llama_32k S={stride} tau={tau}: density {_density(hsel.cnt, p):.3f}, near-tie rows {near} of "
            f"{w.num_heads * p.num_blocks} (every head)")
        if tau == 0.9:
            out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
            torch.cuda.synchronize()
            _report_outputs(f"  llama_32k S={stride} tau=0.9", out, q, k, v, hsel.mask, prm, seed=stride)


# ---------------------------------------------------------------------------
# 64K video (G = 7): every head
# ---------------------------------------------------------------------------
def test_video_64k_every_head():
    w = wl.WORKLOADS["video_64k"]
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p, prm = _params(w)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    _check_any_size(sel, p)
    hsel = _Sel(sel)
    near = _compare_heads(hsel, q, k, prm, range(w.num_heads))
    say(f"video_64k: density {_density(hsel.cnt, p):.3f}, near-tie rows {near} of {w.num_heads * p.num_blocks} "
        f"(every head)")
    _report_outputs("  video_64k", out, q, k, v, hsel.mask, prm, seed=64)


# ---------------------------------------------------------------------------
# 128K (the benchmarked workload): every head, one test per KV group
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def llama_128k():
    """The benchmarked workload run through the same calls and buffers bench.py
    times (workspace-held scores, per-call schedule workspace), plus a run
    that returns the scores; both selections must be identical.  Everything
    the checks need is copied to the host and the device memory released."""
    w = wl.headline()
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p, prm = _params(w)
    ws = rra.alloc_workspace(p)
    sel = rra.Selection(*rra._lib._selection_buffers(p, qd.device), None)
    rra.estimate(p, qd, kd, workspace=ws, out=sel)
    out = torch.empty_like(qd)
    rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)
    score = torch.empty((1, p.num_heads, p.num_blocks, p.num_blocks), dtype=torch.float32, device=qd.device)
    sel2 = rra.estimate(p, qd, kd, out=rra.Selection(*rra._lib._selection_buffers(p, qd.device), score))
    torch.cuda.synchronize()
    assert torch.equal(sel.mask, sel2.mask) and torch.equal(sel.cnt, sel2.cnt)
    listed = torch.arange(p.num_blocks, device=qd.device) < sel.cnt.unsqueeze(-1)  # entries past cnt are unwritten
    assert torch.equal(sel.idx[listed], sel2.idx[listed])
    _check_any_size(sel2, p)
    hsel = _Sel(sel2)
    out_h = out.cpu()
    del qd, kd, vd, ws, sel, sel2, out, score
    torch.cuda.empty_cache()
    say(f"llama_128k: density {_density(hsel.cnt, p):.4f}")
    return w, p, prm, q, k, v, hsel, out_h


@pytest.mark.parametrize("group", range(8))
def test_llama_128k_masks_every_head(llama_128k, group):
    w, p, prm, q, k, v, hsel, _ = llama_128k
    heads = range(group * prm.group, (group + 1) * prm.group)
    near = _compare_heads(hsel, q, k, prm, heads)
    say(f"llama_128k KV group {group} (heads {heads.start}-{heads.stop - 1}): near-tie rows {near} of "
        f"{len(heads) * p.num_blocks}")


def test_llama_128k_outputs(llama_128k):
    w, p, prm, q, k, v, hsel, out_h = llama_128k
    _report_outputs("llama_128k", out_h, q, k, v, hsel.mask, prm, seed=128)


# ---------------------------------------------------------------------------
# Longest rows and ragged lengths
# ---------------------------------------------------------------------------
def test_max_blocks_4096():
    """Nb = 4096 key blocks (the longest row the selection holds), one head, S = Bk."""
    L, d, S, Bk = 4096 * 128, 128, 128, 128
    q, k, v = wl.make_random(1, 1, 1, L, d, seed=3, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(1, 1, 1, L, d, S, Bk, 0.9)
    prm = orc.Params(1, 1, 1, L, d, S, Bk, float(np.float32(0.9)), True)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    _check_any_size(sel, p)
    hsel = _Sel(sel)
    near = _compare_heads(hsel, q, k, prm, [0])
    say(f"Nb=4096: near-tie rows {near}, mean count {sel.cnt.float().mean().item():.1f}")
    e = check_rows_by_head(out, q, k, v, hsel.mask, prm, [(0, 0, 4095), (0, 0, 2048), (0, 0, 17)])
    assert e["err"] <= OUT_ATOL, e


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_32k_every_head(causal):
    """L = 32768 + 77 (last block of 77 tokens), every head's mask and 64
    seeded output rows against the oracle."""
    L, H, Hkv, d, S, Bk, tau = 32768 + 77, 8, 2, 128, 16, 128, 0.9
    q, k, v = wl.make_random(1, H, Hkv, L, d, seed=11, scale=1.2, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(1, H, Hkv, L, d, S, Bk, tau, causal=causal)
    prm = orc.Params(1, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True, causal=causal)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    hsel = _Sel(sel)
    near = _compare_heads(hsel, q, k, prm, range(H))
    say(f"ragged 32K+77 causal={causal}: near-tie rows {near} of {H * p.num_blocks}")
    _report_outputs(f"  ragged 32K+77 causal={causal}", out, q, k, v, hsel.mask, prm, seed=77)


def test_concurrent_streams_match_sequential():
    """The library keeps no mutable global state: the same calls on two streams
    at once give bitwise the results of running them one after the other."""
    w = wl.WORKLOADS["llama_8k"]
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p1 = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, 16, w.block, 0.9)
    p2 = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, 8, w.block, 0.8)
    ref = []
    for p in (p1, p2):
        sel = rra.estimate(p, qd, kd)
        ref.append((sel.mask.clone(), rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt).clone()))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
    got = [None, None]
    torch.cuda.synchronize()
    for rep in range(3):
        for j, (p, s) in enumerate(zip((p1, p2), streams)):
            with torch.cuda.stream(s):
                sel = rra.estimate(p, qd, kd)
                got[j] = (sel.mask, rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt))
        torch.cuda.synchronize()
        for j in range(2):
            assert torch.equal(got[j][0], ref[j][0]) and torch.equal(got[j][1], ref[j][1]), (rep, j)


def test_calls_on_a_side_stream_match_the_current_stream():
    """stream= another stream than the current one: the binding allocates the
    call's workspaces and outputs on that stream, so work queued meanwhile on
    the current stream (allocations filled with NaN) cannot take their bytes
    while the kernels run.  Results bitwise equal to the current-stream ones."""
    B, H, Hkv, L, d, S, Bk, tau = 1, 8, 2, 8192, 128, 16, 128, 0.9
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=21, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    sel = rra.estimate(p, qd, kd, return_score=True)
    ref = (sel.score.clone(), sel.mask.clone(), rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt).clone(),
           rra.dense_attn(p, qd, kd, vd).clone())
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    cur = torch.cuda.current_stream()
    nbytes = rra.workspace_size(p)
    for rep in range(3):
        side.wait_stream(cur)
        s2 = rra.estimate(p, qd, kd, return_score=True, stream=side)
        o2 = rra.sparse_attn(p, qd, kd, vd, s2.idx, s2.cnt, stream=side)
        d2 = rra.dense_attn(p, qd, kd, vd, stream=side)
        for _ in range(4):  # churn the current stream's pool while the side stream runs
            torch.empty(nbytes // 4 + 1024, dtype=torch.float32, device="cuda").fill_(float("nan"))
            torch.empty(4096, dtype=torch.uint8, device="cuda").fill_(0xFF)
        cur.wait_stream(side)
        torch.cuda.synchronize()
        got = (s2.score, s2.mask, o2, d2)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
