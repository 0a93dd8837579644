"""GPU vs CPU-oracle parity of every step, through the C ABI (needs gfx950).

Bars: bit-exact for the bf16 cast, the aggregated keys and the selections
made from identical block scores; block scores within 1e-5 absolute; masks
bit-exact except near-tie rows, which must still be valid Top-tau sets;
attention outputs within 1e-2 max-abs, computed on the GPU's own mask.
"""
import ctypes
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
                     out_err, seeded_rows, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rra.lib()  # raises if librra.so is missing: there is no fallback


def say(*a):
    print(*a, flush=True)


# Small shapes covering every kernel template: (name, B, H, Hkv, L, d, S, Bk, tau)
SMALL = [
    ("d128_bk128_s16", 1, 8, 2, 2048, 128, 16, 128, 0.9),
    ("d128_bk128_s4_r32", 1, 4, 1, 1024, 128, 4, 128, 0.9),
    ("d128_bk128_s32_r4", 1, 8, 2, 2048, 128, 32, 128, 0.8),
    ("d128_bk128_s64_r2", 1, 4, 2, 2048, 128, 64, 128, 0.9),
    ("d128_bk128_s128_r1", 1, 4, 2, 2048, 128, 128, 128, 0.95),
    ("d64_bk64_s8_b2", 2, 4, 1, 1024, 64, 8, 64, 0.9),
    ("d128_bk64_s8", 1, 4, 2, 1024, 128, 8, 64, 0.9),
    ("d64_bk128_s8_r16", 1, 4, 4, 1024, 64, 8, 128, 0.9),
    ("g7_two_row_tiles", 1, 14, 2, 1024, 128, 16, 128, 0.95),
    ("ragged_tail_nb9", 1, 4, 1, 1152, 128, 16, 128, 0.9),
    ("single_block", 1, 4, 2, 128, 128, 16, 128, 0.9),
    ("three_blocks_ns24", 1, 4, 4, 384, 128, 16, 128, 0.7),
]


def _small_inputs(case, seed=0):
    name, B, H, Hkv, L, d, S, Bk, tau = case
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=seed, scale=1.5, diag=1.0)
    prm = orc.Params(B, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    return prm, p, q, k, v


def test_cast_matches_torch_rne():
    g = torch.Generator().manual_seed(3)
    x = (torch.randn(1 << 20, generator=g) * torch.exp(torch.randn(1 << 20, generator=g) * 8)).float()
    x[:7] = torch.tensor([0.0, -0.0, 1.0, 1.00390625, 1.01171875, float("inf"), -3.5])  # incl. ties
    for n in (x.numel(), x.numel() - 5, 3):
        xs = x[:n].contiguous().cuda()
        got = rra.cast_f32_to_bf16(xs)
        torch.cuda.synchronize()
        ref = x[:n].to(torch.bfloat16)
        assert torch.equal(got.cpu().view(torch.int16), ref.view(torch.int16))
        # the oracle's own rounding, written from the bf16 definition (finite values; -0.0 kept by sign)
        fin = torch.isfinite(x[:n])
        o = orc.bf16_round(x[:n][fin].double().numpy())
        assert np.array_equal(to_f64(got.cpu()[fin]), o)
        assert torch.equal(torch.signbit(got.cpu()[fin]), torch.signbit(x[:n][fin]))


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_cases_all_steps(case):
    say("case", case)
    prm, p, q, k, v = _small_inputs(case)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)
    # a1: aggregated keys, bit-exact
    kagg = rra.stride_aggregate(p, kd)
    for b in range(prm.batch):
        for g in range(prm.num_kv_heads):
            ref = orc.aggregate_keys(kn[b, g], prm.stride, "bf16")
            assert np.array_equal(to_f64(kagg[b, g]), ref)
    # a2-a5: block scores
    score = rra.block_scores(p, qd, kagg)
    m_or = orc.block_scores(qn, kn, prm)
    err = float(np.max(np.abs(to_f64(score) - m_or)))
    say("  block score max-abs", err)
    assert err <= SCORE_ATOL
    # a6 on identical scores: bit-exact
    mask, idx, cnt = rra.top_tau(p, score)
    torch.cuda.synchronize()
    sc64 = to_f64(score)
    omask, oidx, ocnt = orc.select_blocks(sc64, prm)
    assert np.array_equal(mask.cpu().numpy(), omask)
    assert np.array_equal(cnt.cpu().numpy(), ocnt)
    idx_np = idx.cpu().numpy()
    for b in range(prm.batch):
        for h in range(prm.num_heads):
            for i in range(prm.num_blocks):
                assert np.array_equal(idx_np[b, h, i, :ocnt[b, h, i]], oidx[b, h, i, :ocnt[b, h, i]])
    # whole estimator vs the oracle's own masses (near-tie rule)
    sel = rra.estimate(p, qd, kd, return_score=True)
    torch.cuda.synchronize()
    assert torch.equal(sel.score, score)
    checked, near, bad = compare_masks(sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(),
                                       m_or, prm)
    say(f"  mask rows {checked}, near-tie rows {near}, bad {len(bad)}")
    assert not bad, bad[:5]
    # a7: sparse attention on the GPU's mask, every row
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    gm = sel.mask.cpu().numpy()
    o_ref = orc.block_sparse_attention(qn, kn, vn, gm, prm)
    err = out_err(to_f64(out), o_ref)
    say("  sparse attn max-abs", err, "raw", float(np.max(np.abs(to_f64(out) - o_ref))))
    assert err <= OUT_ATOL
    # a8: dense attention
    dense = rra.dense_attn(p, qd, kd, vd)
    torch.cuda.synchronize()
    d_ref = orc.dense_attention(qn, kn, vn, prm)
    err = out_err(to_f64(dense), d_ref)
    say("  dense attn max-abs", err, "raw", float(np.max(np.abs(to_f64(dense) - d_ref))))
    assert err <= OUT_ATOL


RR_CASES = [("layer", 5, 0), ("hybrid", 11, 0), ("none", 0, 3), ("none", 0, -1), ("head", 9, 0)]


@pytest.mark.parametrize("shape", [SMALL[0], SMALL[5], SMALL[8]], ids=[SMALL[0][0], SMALL[5][0], SMALL[8][0]])
@pytest.mark.parametrize("rr", RR_CASES, ids=[f"{m}_l{l0}_c{c}" for m, l0, c in RR_CASES])
def test_round_robin_variants(shape, rr):
    """§4.3 round-robin strategies: block scores and masks against the oracle
    (offset -1 stands for S - 1, the last position of every stride)."""
    mode, layer, fixed = rr
    name, B, H, Hkv, L, d, S, Bk, tau = shape
    fixed = S - 1 if fixed < 0 else fixed
    q, k, _ = wl.make_random(B, H, Hkv, L, d, seed=4, scale=1.5, diag=1.0)
    prm = orc.Params(B, H, Hkv, L, d, S, Bk, float(np.float32(tau)), True, rr_mode=mode, rr_layer=layer,
                     rr_fixed=fixed)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau, rr_mode=mode, rr_layer=layer, rr_offset=fixed)
    say("rr case", name, mode, layer, fixed)
    qd, kd = q.cuda(), k.cuda()
    sel = rra.estimate(p, qd, kd, return_score=True)
    torch.cuda.synchronize()
    m_or = orc.block_scores(to_f64(q), to_f64(k), prm)
    err = float(np.max(np.abs(to_f64(sel.score) - m_or)))
    assert err <= SCORE_ATOL, err
    checked, near, bad = compare_masks(sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(),
                                       m_or, prm)
    say(f"  score err {err:.1e}, mask rows {checked}, near-tie rows {near}")
    assert not bad, bad[:5]
    # the strategy matters: head-RR scores differ unless the offsets coincide
    p_head = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    sel_head = rra.estimate(p_head, qd, kd, return_score=True)
    torch.cuda.synchronize()
    same_offsets = all(orc.rr_offset(h, S, mode, layer, fixed) == h % S for h in range(H))
    assert torch.equal(sel.score, sel_head.score) == same_offsets


def test_tiny_workload_end_to_end():
    w = wl.WORKLOADS["tiny_1k"]
    q32, k32, v32 = wl.make_inputs(w)
    prm = oracle_params(w)
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
    qd = rra.cast_f32_to_bf16(q32.cuda())
    kd = rra.cast_f32_to_bf16(k32.cuda())
    vd = rra.cast_f32_to_bf16(v32.cuda())
    qn, kn, vn = to_f64(q32.to(torch.bfloat16)), to_f64(k32.to(torch.bfloat16)), to_f64(v32.to(torch.bfloat16))
    assert np.array_equal(to_f64(qd), qn) and np.array_equal(to_f64(kd), kn)
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    torch.cuda.synchronize()
    m_or = orc.block_scores(qn, kn, prm)
    assert float(np.max(np.abs(to_f64(sel.score) - m_or))) <= SCORE_ATOL
    checked, near, bad = compare_masks(sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(),
                                       m_or, prm)
    say(f"tiny_1k mask rows {checked}, near-tie {near}")
    assert not bad
    o_ref = orc.block_sparse_attention(qn, kn, vn, sel.mask.cpu().numpy(), prm)
    assert out_err(to_f64(out), o_ref) <= OUT_ATOL


def test_llama_8k_masks_full_outputs_sampled():
    w = wl.WORKLOADS["llama_8k"]
    q, k, v = wl.make_inputs(w)
    prm = oracle_params(w)
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sel = rra.estimate(p, qd, kd, return_score=True)
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    dense = rra.dense_attn(p, qd, kd, vd)
    torch.cuda.synchronize()
    qn, kn, vn = to_f64(q), to_f64(k), to_f64(v)
    m_or = orc.block_scores(qn, kn, prm)
    err = float(np.max(np.abs(to_f64(sel.score) - m_or)))
    gm = sel.mask.cpu().numpy()
    checked, near, bad = compare_masks(gm, sel.cnt.cpu().numpy(), sel.idx.cpu().numpy(), m_or, prm)
    dens = sel.cnt.sum().item() / (prm.num_heads * prm.num_blocks * (prm.num_blocks + 1) / 2)
    say(f"llama_8k score err {err:.2e} rows {checked} near-tie {near} density {dens:.3f}")
    assert err <= SCORE_ATOL
    assert not bad, bad[:5]
    rows = seeded_rows(8, 1, 32, 64, 64)
    e_sp = check_rows_by_head(out, q, k, v, gm, prm, rows)
    full = np.broadcast_to(np.tril(np.ones((64, 64), dtype=np.uint8)), gm.shape)
    e_dn = check_rows_by_head(dense, q, k, v, full, prm, rows)
    say(f"  64 seeded output rows: sparse err {e_sp['err']:.2e} (raw {e_sp['max_abs']:.2e}, rel {e_sp['max_rel']:.2e}), "
        f"dense err {e_dn['err']:.2e} (raw {e_dn['max_abs']:.2e}, rel {e_dn['max_rel']:.2e})")
    assert e_sp["err"] <= OUT_ATOL and e_dn["err"] <= OUT_ATOL


def test_tau_one_sparse_equals_dense_bitwise_and_determinism():
    case = ("d128_bk128_s16", 1, 8, 2, 2048, 128, 16, 128, 1.0)
    prm, p, q, k, v = _small_inputs(case, seed=5)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    sel = rra.estimate(p, qd, kd)
    torch.cuda.synchronize()
    nb = prm.num_blocks
    assert torch.equal(sel.cnt.cpu(), torch.arange(1, nb + 1, dtype=torch.int32).expand(1, 8, nb))
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    dense = rra.dense_attn(p, qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)
    # determinism of the whole path
    p2 = rra.make_params(1, 8, 2, 2048, 128, 16, 128, 0.9)
    s1 = rra.estimate(p2, qd, kd, return_score=True)
    o1 = rra.sparse_attn(p2, qd, kd, vd, s1.idx, s1.cnt)
    s2 = rra.estimate(p2, qd, kd, return_score=True)
    o2 = rra.sparse_attn(p2, qd, kd, vd, s2.idx, s2.cnt)
    torch.cuda.synchronize()
    assert torch.equal(s1.score, s2.score) and torch.equal(s1.mask, s2.mask) and torch.equal(o1, o2)


def test_protect_last_flag_and_empty_problem():
    case = ("d128_bk128_s16", 1, 4, 2, 2048, 128, 16, 128, 0.5)
    prm, p, q, k, v = _small_inputs(case, seed=6)
    qd, kd = q.cuda(), k.cuda()
    sel = rra.estimate(p, qd, kd)
    p0 = rra.make_params(1, 4, 2, 2048, 128, 16, 128, 0.5, protect_last=False)
    sel0 = rra.estimate(p0, qd, kd)
    torch.cuda.synchronize()
    nb = prm.num_blocks
    assert torch.all(sel.cnt[..., -1] == nb)
    assert torch.all(sel0.cnt[..., -1] < nb)
    assert torch.equal(sel.cnt[..., :-1], sel0.cnt[..., :-1])
    # empty problem: nothing to do, nothing written
    pe = rra.make_params(0, 4, 2, 2048, 128, 16, 128, 0.5)
    assert rra.lib().rra_dense_attn(ctypes.byref(pe), None, None, None, None, None, 0, None) == 0
    e = torch.empty(0, 4, 2048, 128, dtype=torch.bfloat16, device="cuda")
    ek = torch.empty(0, 2, 2048, 128, dtype=torch.bfloat16, device="cuda")
    assert rra.dense_attn(pe, e, ek, ek).shape == e.shape


def test_invalid_arguments_raise():
    p = rra.make_params(1, 4, 2, 1024, 96, 16, 128, 0.9)  # d = 96 is not built
    q = torch.zeros(1, 4, 1024, 96, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 1024, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rra.RRAError) as ei:
        rra.dense_attn(p, q, k, k)
    assert ei.value.code == 2
    p = rra.make_params(1, 4, 2, 1024, 128, 16, 128, 0.9)
    q = torch.zeros(1, 4, 1024, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        rra.estimate(p, q, q)  # k has the wrong shape: caught before the library
