"""The attention kernel's two schedules give bitwise the same output (needs gfx950).

With a workspace, rra_sparse_attn / rra_dense_attn run a fixed set of
resident workgroups that pop (b, h, I) rows from per-XCD queues and steal
from the other queues; without one, every row is its own workgroup.  Each
row is computed by the same code either way, so outputs must be identical
bit for bit: on every kernel template (d 64/128, Bk 64/128), ragged and
non-causal shapes, sparse and dense, with rows enough to exceed the resident
workgroups (so the queues and the stealing run).  The workspace's contents on
entry must not matter, one workspace serves consecutive calls, and a short
one is refused before anything is launched.  Rows whose list is empty
(cnt = 0) come out as zeros without disturbing the others.  (Agreement of
these outputs with the oracle is the business of the other parity tests.)
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


def say(*a):
    print(*a, flush=True)


# (name, B, H, Hkv, L, d, S, Bk, tau, causal): rows B*H*ceil(L/Bk) >= 2048
CASES = [
    ("d128_bk128", 1, 32, 8, 8192, 128, 16, 128, 0.9, True),
    ("d128_bk128_ragged_noncausal", 1, 16, 4, 16384 + 77, 128, 16, 128, 0.8, False),
    ("d128_bk64", 1, 8, 2, 16384, 128, 8, 64, 0.9, True),
    ("d64_bk128_b2", 2, 16, 4, 8192 + 5, 64, 16, 128, 0.9, True),
    ("d64_bk64_noncausal", 1, 8, 8, 16384, 64, 8, 64, 0.9, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_dynamic_equals_static(case):
    name, B, H, Hkv, L, d, S, Bk, tau, causal = case
    say("case", case)
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=21, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, tau, causal=causal)
    assert B * H * p.num_blocks >= 2048
    sel = rra.estimate(p, qd, kd)
    ws = torch.full((rra.attn_workspace_size(p),), 0xFF, dtype=torch.uint8, device="cuda")  # garbage on entry
    sp_static = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, schedule="static")
    sp_dyn = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, workspace=ws)
    sp_dyn2 = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, workspace=ws)  # the same workspace again
    dn_static = rra.dense_attn(p, qd, kd, vd, schedule="static")
    dn_dyn = rra.dense_attn(p, qd, kd, vd, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(sp_dyn, sp_static)
    assert torch.equal(sp_dyn2, sp_static)
    assert torch.equal(dn_dyn, dn_static)
    assert not torch.equal(sp_static, dn_static)  # the sparse lists did skip blocks


def test_llama_128k_rows_schedule_identical():
    """The bench configuration: the whole 128K launch, dynamic vs static, bitwise."""
    w = wl.WORKLOADS["llama_128k"]
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    del q, k, v
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
    sel = rra.estimate(p, qd, kd)
    a = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt)
    b = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, schedule="static")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_short_workspace_is_refused():
    p = rra.make_params(1, 4, 2, 1024, 64, 8, 64, 0.9)
    q = torch.zeros((1, 4, 1024, 64), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, 1024, 64), dtype=torch.bfloat16, device="cuda")
    short = torch.empty(rra.attn_workspace_size(p) - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(rra.RRAError) as ei:
        rra.dense_attn(p, q, kv, kv, workspace=short)
    assert ei.value.code == 3
    n = ctypes.c_size_t(0)
    assert rra.lib().rra_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0 and n.value == 1024


@pytest.mark.parametrize("schedule", ["dynamic", "static"])
def test_empty_lists_give_zero_rows(schedule):
    """cnt = 0 rows (no block selected) come out as zeros; every other row is
    bitwise what it is with the lists untouched."""
    B, H, Hkv, L, d, S, Bk = 1, 8, 2, 4096 + 40, 128, 16, 128
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=5, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, 0.9)
    sel = rra.estimate(p, qd, kd)
    ref = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, schedule=schedule)
    cnt = sel.cnt.clone()
    zero_rows = [(0, 0, 0), (0, 3, 7), (0, 5, p.num_blocks - 1), (0, 7, 20)]
    for b, h, i in zero_rows:
        cnt[b, h, i] = 0
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, cnt, schedule=schedule)
    torch.cuda.synchronize()
    keep = torch.ones((B, H, L), dtype=torch.bool, device="cuda")
    for b, h, i in zero_rows:
        rows = slice(i * Bk, min((i + 1) * Bk, L))
        assert torch.count_nonzero(out[b, h, rows]).item() == 0
        keep[b, h, rows] = False
    assert torch.equal(out[keep], ref[keep])


def test_workspaces_of_any_dtype_are_sized_in_bytes():
    """A float32 workspace of the required bytes serves estimate and sparse
    attention exactly like a uint8 one; host-memory workspaces are refused."""
    B, H, Hkv, L, d, S, Bk = 1, 8, 2, 2048, 128, 16, 128
    q, k, v = wl.make_random(B, H, Hkv, L, d, seed=9, scale=1.5, diag=1.0)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(B, H, Hkv, L, d, S, Bk, 0.9)
    ref = rra.estimate(p, qd, kd)
    ws32 = torch.empty((rra.workspace_size(p) + 3) // 4, dtype=torch.float32, device="cuda")
    sel = rra.estimate(p, qd, kd, workspace=ws32)
    a32 = torch.empty((rra.attn_workspace_size(p) + 3) // 4, dtype=torch.float32, device="cuda")
    out = rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, workspace=a32)
    want = rra.sparse_attn(p, qd, kd, vd, ref.idx, ref.cnt)
    torch.cuda.synchronize()
    assert torch.equal(sel.mask, ref.mask) and torch.equal(sel.cnt, ref.cnt)
    assert torch.equal(out, want)
    with pytest.raises(ValueError):
        rra.estimate(p, qd, kd, workspace=torch.empty(rra.workspace_size(p), dtype=torch.uint8))
    with pytest.raises(ValueError):
        rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, workspace=torch.empty(1024, dtype=torch.uint8))
