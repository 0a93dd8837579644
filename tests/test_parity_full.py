"""GPU vs oracle at the workloads' full sizes (needs gfx950).

The GPU runs every head and row; the oracle checks sampled heads (whole mask
rows) and sampled output rows, which it can compute one by one, plus
properties that hold at any size (score rows sum to 1, masks agree with their
index lists and counts, the protected last row is full).
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
from helpers import OUT_ATOL, SCORE_ATOL, check_output_rows, compare_masks, oracle_params, to_f64  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()


def say(*a):
    print(*a, flush=True)


def _head_scores(q, k, prm, h):
    """Oracle block scores of one query head: [Nb, Nb]."""
    g = h // prm.group
    kagg = orc.aggregate_keys(k[0, g].double().numpy(), prm.stride)
    s = orc.stride_scores(q[0, h].double().numpy(), kagg, prm.stride, h, prm.scale, prm.rr_mode, prm.rr_layer,
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
    assert torch.all(cnt <= i_idx + 1)
    if p.protect_last:
        assert torch.all(cnt[..., -1] == nb)
    tri = torch.triu(torch.ones(nb, nb, dtype=torch.bool, device=cnt.device), 1)
    assert not torch.any(sel.mask.bool() & tri)
    assert not torch.any(score.masked_select(tri.expand_as(score)) != 0)


def _run(w, tau=None, stride=None):
    t = w.tau if tau is None else tau
    s = w.stride if stride is None else stride
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, s, w.block, t)
    return p, oracle_params(w, tau=t, stride=s)


def _mask_parity(sel, q, k, prm, heads):
    gm = sel.mask.cpu().numpy()
    gc = sel.cnt.cpu().numpy()
    gi = sel.idx.cpu().numpy()
    gs = to_f64(sel.score)
    near_total = 0
    for h in heads:
        m_h = _head_scores(q, k, prm, h)
        err = float(np.max(np.abs(gs[0, h] - m_h)))
        assert err <= SCORE_ATOL, (h, err)
        m_full = np.zeros((1, prm.num_heads) + m_h.shape)
        m_full[0, h] = m_h
        checked, near, bad = compare_masks(gm, gc, gi, m_full, prm, heads=[h])
        assert not bad, (h, bad[:3])
        near_total += near
    return near_total


@pytest.fixture(scope="module")
def llama_32k():
    w = wl.WORKLOADS["llama_32k"]
    q, k, v = wl.make_inputs(w)
    return w, q, k, v, q.cuda(), k.cuda(), v.cuda()


@pytest.mark.parametrize("stride", [8, 16, 32])
def test_llama_32k_sweep(llama_32k, stride):
    """All three taus of one stride (the block scores are shared)."""
    w, q, k, v, qd, kd, vd = llama_32k
    heads = [0, 1, 6, 13, 22, 31]  # banded (even) and column (odd) heads, several KV groups
    cache = {}
    for tau in (0.8, 0.9, 0.95):
        p, prm = _run(w, tau=tau, stride=stride)
        sel = rra.estimate(p, qd, kd, return_score=True)
        torch.cuda.synchronize()
        _check_any_size(sel, p)
        gm, gc, gi, gs = sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(), to_f64(sel.score)
        near = 0
        for h in heads:
            if h not in cache:
                cache[h] = _head_scores(q, k, prm, h)
            m_h = cache[h]
            assert float(np.max(np.abs(gs[0, h] - m_h))) <= SCORE_ATOL
            m_full = np.zeros((1, prm.num_heads) + m_h.shape)
            m_full[0, h] = m_h
            _, n_near, bad = compare_masks(gm, gc, gi, m_full, prm, heads=[h])
            assert not bad, (stride, tau, h, bad[:3])
            near += n_near
        dens = sel.cnt.sum().item() / (p.num_heads * p.num_blocks * (p.num_blocks + 1) / 2)
        say(f"llama_32k S={stride} tau={tau}: density {dens:.3f}, near-tie rows {near} of {len(heads) * p.num_blocks}")
    # outputs on the last (tau = 0.95) mask, sampled rows
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    rows = [(0, 1, 255), (0, 6, 100), (0, 31, 17), (0, 0, 0)]
    err = check_output_rows(out, q.double().numpy(), k.double().numpy(), v.double().numpy(), gm, prm, rows)
    say(f"  sampled output err {err:.2e}")
    assert err <= OUT_ATOL


def test_video_64k():
    w = wl.WORKLOADS["video_64k"]
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p, prm = _run(w)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    _check_any_size(sel, p)
    near = _mask_parity(sel, q, k, prm, heads=[0, 6, 7, 20, 27])  # G = 7: both ends of groups
    dens = sel.cnt.sum().item() / (p.num_heads * p.num_blocks * (p.num_blocks + 1) / 2)
    say(f"video_64k: density {dens:.3f}, near-tie rows {near}")
    rows = [(0, 27, 511), (0, 3, 300), (0, 13, 508)]
    err = check_output_rows(out, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                            sel.mask.cpu().numpy(), prm, rows)
    say(f"  sampled output err {err:.2e}")
    assert err <= OUT_ATOL


def test_llama_128k_headline_in_bench_configuration():
    """The benchmarked workload, through the same calls and buffers bench.py uses."""
    w = wl.headline()
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p, prm = _run(w)
    ws = rra.alloc_workspace(p)
    sel = rra.Selection(*rra._lib._selection_buffers(p, qd.device), None)
    rra.estimate(p, qd, kd, workspace=ws, out=sel)
    out = torch.empty_like(qd)
    rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)
    score = torch.empty((1, p.num_heads, p.num_blocks, p.num_blocks), dtype=torch.float32, device=qd.device)
    sel2 = rra.estimate(p, qd, kd, out=rra.Selection(*rra._lib._selection_buffers(p, qd.device), score))
    torch.cuda.synchronize()
    assert torch.equal(sel.mask, sel2.mask) and torch.equal(sel.cnt, sel2.cnt)
    _check_any_size(sel2, p)
    near = _mask_parity(sel2, q, k, prm, heads=[0, 13])
    dens = sel.cnt.sum().item() / (p.num_heads * p.num_blocks * (p.num_blocks + 1) / 2)
    say(f"llama_128k: density {dens:.3f}, near-tie rows {near}")
    rows = [(0, 13, 1023), (0, 0, 700), (0, 31, 64), (0, 7, 0)]
    err = check_output_rows(out, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                            sel.mask.cpu().numpy(), prm, rows)
    say(f"  sampled output err {err:.2e}")
    assert err <= OUT_ATOL


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
    near = _mask_parity(sel, q, k, prm, heads=[0])
    say(f"Nb=4096: near-tie rows {near}, mean count {sel.cnt.float().mean().item():.1f}")
    err = check_output_rows(out, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                            sel.mask.cpu().numpy(), prm, [(0, 0, 4095), (0, 0, 2048)])
    assert err <= OUT_ATOL


@pytest.mark.parametrize("causal", [True, False])
def test_ragged_32k_sampled(causal):
    """L = 32768 + 77 (last block of 77 tokens, plain work order), sampled mask
    rows and output rows against the oracle."""
    L, H, Hkv, d, S, Bk, tau = 32768 + 77, 8, 2, 128, 16, 128, 0.9
    q, k, v = wl.make_random(1, H, Hkv, L, d, seed=11, scale=1.2, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(1, H, Hkv, L, d, S, Bk, tau, causal=causal)
    prm = orc.Params(1, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True, causal=causal)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    near = _mask_parity(sel, q, k, prm, heads=[0, 5])
    nb = p.num_blocks
    rows = [(0, 0, nb - 1), (0, 5, nb - 1), (0, 3, nb // 2), (0, 7, 0)]
    err = check_output_rows(out, q.double().numpy(), k.double().numpy(), v.double().numpy(),
                            sel.mask.cpu().numpy(), prm, rows)
    say(f"ragged 32K+77 causal={causal}: near-tie rows {near}, sampled output err {err:.2e}")
    assert err <= OUT_ATOL


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
