"""The hot path captured in a HIP graph replays bitwise like eager calls (needs gfx950).

rra_estimate (aggregation, scores, Top-tau) and rra_sparse_attn on the dynamic
schedule (its counters are cleared by a kernel, not a memset) are captured
once and replayed several times; between the replays the program runs eager
work of its own (a dense launch on the same workspace, a scribble over the
outputs) and synchronises.  Every replay must reproduce the eager mask, index
lists, counts and output exactly.
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


def test_graph_replays_match_eager():
    w = wl.WORKLOADS["llama_8k"]  # 32 heads x 64 query blocks: more rows than resident workgroups
    q, k, v = wl.make_inputs(w)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
    nb = p.num_blocks
    est_ws = rra.alloc_workspace(p)
    attn_ws = torch.empty(rra.attn_workspace_size(p), dtype=torch.uint8, device="cuda")
    shape = (w.batch, w.num_heads, nb, nb)
    sel = rra.Selection(torch.empty(shape, dtype=torch.uint8, device="cuda"),
                        torch.empty(shape, dtype=torch.int32, device="cuda"),
                        torch.empty(shape[:3], dtype=torch.int32, device="cuda"), None)
    out = torch.empty_like(qd)

    def path():
        rra.estimate(p, qd, kd, workspace=est_ws, out=sel)
        rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out, workspace=attn_ws)

    path()
    torch.cuda.synchronize()
    want = (sel.mask.clone(), sel.idx.clone(), sel.cnt.clone(), out.clone())
    valid = torch.arange(nb, device="cuda").view(1, 1, 1, nb) < want[2].unsqueeze(-1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        path()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    dense = torch.empty_like(qd)
    for rep in range(4):
        # eager work between replays: scribble over the outputs, use the same schedule workspace
        sel.mask.fill_(7)
        sel.idx.fill_(-3)
        sel.cnt.fill_(-3)
        out.fill_(float("nan"))
        rra.dense_attn(p, qd, kd, vd, out=dense, workspace=attn_ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel.mask, want[0]), rep
        assert torch.equal(sel.cnt, want[2]), rep
        assert torch.equal(torch.where(valid, sel.idx, 0), torch.where(valid, want[1], 0)), rep
        assert torch.equal(out, want[3]), rep
