"""rra_estimate_noalloc (intermediates in the library's own device array)
against rra_estimate (caller workspace), through the C ABI (needs gfx950).

The two entry points run the same kernels, so masks, counts, the listed index
entries and the block scores must be bitwise equal.  Calls follow each other
on the shared array with the larger problem first, so the smaller call runs
on the previous call's leftovers.  Outputs start poisoned (NaN / junk) so
every byte compared was written by the call.
"""
import ctypes

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


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _poisoned(p, with_score):
    B, H, nb = p.batch, p.num_heads, p.num_blocks
    return rra.Selection(torch.full((B, H, nb, nb), 0xAB, dtype=torch.uint8, device="cuda"),
                         torch.full((B, H, nb, nb), -7, dtype=torch.int32, device="cuda"),
                         torch.full((B, H, nb), -7, dtype=torch.int32, device="cuda"),
                         torch.full((B, H, nb, nb), float("nan"), device="cuda") if with_score else None)


def _noalloc_c(p, qd, kd, sel):
    """One call of the C entry point itself (ctypes, no binding logic)."""
    return rra.lib().rra_estimate_noalloc(ctypes.byref(p), _ptr(qd), _ptr(kd), _ptr(sel.mask), _ptr(sel.idx),
                                          _ptr(sel.cnt), _ptr(sel.score), None)


def _same(a, b, p):
    assert torch.equal(a.mask, b.mask)
    assert torch.equal(a.cnt, b.cnt)
    listed = torch.arange(p.num_blocks, device="cuda") < a.cnt.unsqueeze(-1)
    assert torch.equal(a.idx[listed], b.idx[listed])
    if a.score is not None and b.score is not None:
        assert torch.equal(a.score, b.score)


# (B, H, Hkv, L, d, S, Bk, tau, causal): each case smaller than the one before
CASES = [
    (1, 32, 8, 32768, 128, 16, 128, 0.9, True),  # array: 4.2 MB of aggregated keys + 8.4 MB of scores
    (2, 4, 1, 3000, 64, 8, 64, 0.8, True),      # ragged, another kernel template
    (1, 4, 2, 1000, 128, 16, 128, 0.95, False),  # ragged, no causal mask
]


@pytest.mark.parametrize("with_score", [False, True])
def test_noalloc_matches_estimate_on_calls_of_decreasing_size(with_score):
    for n, case in enumerate(CASES):
        B, H, Hkv, L, d, S, Bk, tau, causal = case
        print(f"noalloc case {n}: {case}, score {'given' if with_score else 'in the array'}", flush=True)
        q, k, _ = wl.make_random(B, H, Hkv, L, d, seed=30 + n, scale=1.5, diag=1.0)
        qd, kd = q.cuda(), k.cuda()
        p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau, causal=causal)
        ref = rra.estimate(p, qd, kd, return_score=True)
        got = _poisoned(p, with_score)
        assert _noalloc_c(p, qd, kd, got) == 0
        got2 = rra.estimate_noalloc(p, qd, kd, _poisoned(p, with_score))  # through the binding as well
        torch.cuda.synchronize()
        _same(got, ref, p)
        _same(got2, ref, p)


def test_noalloc_full_size_with_scores_given_and_limit():
    """The 128K layer (32 query / 8 KV heads, S = 16): with `score` given only
    the aggregated keys (16.8 MB) use the array, and the result equals
    rra_estimate's; with `score` NULL the block scores (134 MB) would not
    fit, and the call is refused before anything is enqueued."""
    B, H, Hkv, L, d, S, Bk, tau = 1, 32, 8, 131072, 128, 16, 128, 0.9
    g = torch.Generator(device="cuda").manual_seed(5)
    qd = torch.randn((B, H, L, d), generator=g, device="cuda").to(torch.bfloat16)
    kd = torch.randn((B, Hkv, L, d), generator=g, device="cuda").to(torch.bfloat16)
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau)
    ref = rra.estimate(p, qd, kd, return_score=True)
    got = _poisoned(p, True)
    assert _noalloc_c(p, qd, kd, got) == 0
    torch.cuda.synchronize()
    _same(got, ref, p)
    refused = _poisoned(p, False)
    assert _noalloc_c(p, qd, kd, refused) == rra._lib.RRA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(refused.cnt.min()) == -7 and int(refused.cnt.max()) == -7  # nothing was written
    # a smaller call after the refused one still matches
    p2 = rra.make_params(1, 4, 1, 4096, 128, 16, 128, 0.9)
    q2, k2 = qd[:, :4, :4096].contiguous(), kd[:, :1, :4096].contiguous()
    ref2 = rra.estimate(p2, q2, k2, return_score=True)
    got2 = _poisoned(p2, False)
    assert _noalloc_c(p2, q2, k2, got2) == 0
    torch.cuda.synchronize()
    _same(got2, ref2, p2)
