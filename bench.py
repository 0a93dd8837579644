#!/usr/bin/env python3
"""Benchmark of RRAttention block-sparse causal prefill on one MI355X.

One step = the whole hot path on one attention layer of the headline
workload (Llama-3-8B shape: 32 query heads, 8 KV heads, d = 128, L = 131072,
S = 16, Bk = 128, tau = 0.9): rra_estimate (stride aggregation, round-robin
sampled scores + stride softmax + block pooling, Top-tau selection) followed
by rra_sparse_attn.  Inputs are seeded synthetic bf16 tensors already resident
in HBM when the timed region starts.  The dense causal flash attention of the
same library is timed on the same inputs for the speedup.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--workload llama_128k]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
COPY_BYTES = 256 << 20  # plain device copy used to calibrate the HBM byte counters


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(q, k, v, sel_mask, cnt, w, f_dense, n_heads_sample=4, n_rows_sample=16):
    """The fp64 CPU oracle on a bounded sample of the same workload.

    Times the oracle's estimator on n_heads_sample query heads (full length)
    and its attention on n_rows_sample sampled (head, query block) rows (on the
    GPU's mask), then extrapolates to the whole layer: the estimator by head
    count, the attention by the number of selected key blocks."""
    import numpy as np
    import torch
    from oracle import rra_oracle as orc
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max([d.get("num_threads", 1) for d in info] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    prm = orc.Params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block,
                     float(np.float32(w.tau)), True)
    nb = prm.num_blocks
    t0 = time.perf_counter()
    for h in range(n_heads_sample):
        g = h // prm.group
        kagg = orc.aggregate_keys(k[0, g].double().numpy(), prm.stride)
        s = orc.stride_scores(q[0, h].double().numpy(), kagg, prm.stride, h, prm.scale)
        m = orc.pool_blocks(orc.stride_softmax(s), prm.strides_per_block)
        for i in range(nb):
            orc.top_tau_row(m[i], i, prm.tau, i == nb - 1)
    t_est = (time.perf_counter() - t0) / n_heads_sample * w.num_heads * w.batch
    rng = np.random.default_rng(0)
    rows = [(0, int(rng.integers(0, w.num_heads)), int(rng.integers(nb // 2, nb))) for _ in range(n_rows_sample)]
    t_attn_sample = 0.0
    blocks_sample = 0
    for (b, h, i) in rows:
        g = h // prm.group
        sub_q = q[b:b + 1, h:h + 1].double().numpy()
        sub_k = k[b:b + 1, g:g + 1].double().numpy()
        sub_v = v[b:b + 1, g:g + 1].double().numpy()
        one = orc.Params(1, 1, 1, prm.seq_len, prm.head_dim, prm.stride, prm.block, prm.tau, True)
        mrow = sel_mask[b:b + 1, h:h + 1]
        t1 = time.perf_counter()
        orc.attention_rows(sub_q, sub_k, sub_v, mrow, one, 0, 0, i)
        t_attn_sample += time.perf_counter() - t1
        blocks_sample += int(cnt[b, h, i])
    t_attn = t_attn_sample / max(blocks_sample, 1) * float(cnt.sum())
    t_total = t_est + t_attn
    return {
        "value": f_dense / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: estimator on {n_heads_sample} of {w.num_heads} heads at full length "
                   f"({time.perf_counter() - t0:.1f} s wall incl. attention), attention on {n_rows_sample} sampled "
                   f"(head, query-block) rows ({blocks_sample} key blocks); extrapolated to the whole layer "
                   f"by heads and by selected blocks: {t_total:.0f} s per step"),
        "extrapolated_s_per_step": t_total,
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["bench", "profile", "power", "selection", "workloads"], default="bench",
                    help="profile: one estimate, --steps sparse-attention launches, one dense launch and a "
                         "256 MiB device copy (HBM-counter calibration); prints a short summary only. "
                         "power: socket power (amd-smi) while sparse attention, dense attention and the "
                         "MFMA probe each run back to back for --power-secs seconds. "
                         "selection: precision / recall / F1 and kept attention mass of the estimated "
                         "selections (round-robin variants, several S and tau) against the exact Top-tau "
                         "selection, one JSON line per point. workloads: estimate / sparse / dense times and "
                         "density of every bf16 workload at its own settings, one JSON line each")
    ap.add_argument("--power-secs", type=float, default=6.0)
    ap.add_argument("--traffic-json", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "profiles", "traffic_sparse_attn_llama_128k.json"))
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the path shards by KV group "
              "with no exchange, so run one process per GPU instead.", file=sys.stderr)
        return 2

    import torch

    import dynamic_block_sparse_sample_amd as rra
    from dynamic_block_sparse_sample_amd import workloads as wl

    rra.lib()  # fail loudly without the HIP library
    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    if args.mode == "selection":
        for line in selection_report(args.workload):
            print(json.dumps(line), flush=True)
        return 0
    if args.mode == "workloads":
        for line in workloads_report():
            print(json.dumps(line), flush=True)
        return 0
    w = wl.WORKLOADS[args.workload]
    if w.fp32_inputs:
        log("pick a bf16 workload for the benchmark")
        return 2
    log(f"[bench] generating {w.name} inputs (seed {w.seed})")
    t0 = time.time()
    q, k, v = wl.make_inputs(w)
    log(f"[bench] generated in {time.time() - t0:.1f}s; copying to the GPU")
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
    nb = p.num_blocks
    ws = rra.alloc_workspace(p, dev)
    sel = rra.Selection(*rra._lib._selection_buffers(p, dev), None)
    out = torch.empty_like(qd)
    dense_out = torch.empty_like(qd)
    torch.cuda.synchronize()

    def step():
        rra.estimate(p, qd, kd, workspace=ws, out=sel)
        rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)

    if args.mode == "profile":
        rra.estimate(p, qd, kd, workspace=ws, out=sel)
        for _ in range(args.steps):
            rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)
        rra.dense_attn(p, qd, kd, vd, out=dense_out)
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # calibration: reads and writes exactly COPY_BYTES
        torch.cuda.synchronize()
        log(f"[bench] profile run done: sum(cnt) = {int(sel.cnt.sum())}, copy {COPY_BYTES} B")
        return 0

    if args.mode == "power":
        rra.estimate(p, qd, kd, workspace=ws, out=sel)
        torch.cuda.synchronize()
        f_sel = 4.0 * w.head_dim * w.block * w.block * int(sel.cnt.sum())
        f_full = 4.0 * w.head_dim * w.block * w.block * p.batch * p.num_heads * nb * (nb + 1) // 2
        print(json.dumps(power_report(
            lambda: rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out), f_sel,
            lambda: rra.dense_attn(p, qd, kd, vd, out=dense_out), f_full, args.power_secs)), flush=True)
        return 0

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps")
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    start, end = E(), E()
    sp_ev = [(E(), E()) for _ in range(args.steps)]
    est_ev = [(E(), E()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        est_ev[i][0].record()
        rra.estimate(p, qd, kd, workspace=ws, out=sel)
        est_ev[i][1].record()
        sp_ev[i][0].record()
        rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)
        sp_ev[i][1].record()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    sp_times = sorted(a.elapsed_time(b) for a, b in sp_ev)
    t_sp = sum(sp_times) / args.steps
    t_est = sum(a.elapsed_time(b) for a, b in est_ev) / args.steps

    # per-kernel breakdown of the estimator (same buffers)
    kagg = ws[: p.batch * p.num_kv_heads * p.num_strides * p.head_dim * 2].view(torch.bfloat16).view(
        p.batch, p.num_kv_heads, p.num_strides, p.head_dim)
    score = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=dev)
    reps = 5
    brk = {}
    for name, fn in [("stride_aggregate", lambda: rra.stride_aggregate(p, kd, kagg)),
                     ("block_scores", lambda: rra.block_scores(p, qd, kagg, score)),
                     ("top_tau", lambda: rra.top_tau(p, score, sel.mask, sel.idx, sel.cnt))]:
        fn()
        a, b = E(), E()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        brk[name] = a.elapsed_time(b) / reps

    log(f"[bench] dense baseline x{args.dense_reps}")
    rra.dense_attn(p, qd, kd, vd, out=dense_out)
    torch.cuda.synchronize()
    a, b = E(), E()
    a.record()
    for _ in range(args.dense_reps):
        rra.dense_attn(p, qd, kd, vd, out=dense_out)
    b.record()
    torch.cuda.synchronize()
    t_dense = a.elapsed_time(b) / args.dense_reps

    # the timed steps left the selection of this input in sel
    cnt = sel.cnt.cpu()
    sum_cnt = int(cnt.sum())
    causal_blocks = p.batch * p.num_heads * nb * (nb + 1) // 2
    density = sum_cnt / causal_blocks
    # per head (min / median / max), and without the protected last row
    per_head = (cnt.double().sum(-1) / (nb * (nb + 1) / 2)).flatten().sort().values
    dens_no_last = (sum_cnt - int(cnt[..., -1].sum())) / (p.batch * p.num_heads * nb * (nb - 1) / 2) if nb > 1 else 1.0
    # exact unmasked work: a selected diagonal block has Bk (Bk + 1) / 2 causal (t, u) pairs, not Bk^2
    diag_sel = int(torch.diagonal(sel.mask, dim1=-2, dim2=-1).long().sum())
    L, d, Bk = w.seq_len, w.head_dim, w.block
    f_dense = 4.0 * d * w.batch * w.num_heads * L * (L + 1) / 2
    f_sel = 4.0 * d * Bk * Bk * sum_cnt
    achieved = f_sel / (t_sp * 1e-3) / 1e12
    value = f_dense / (ms_step * 1e-3) / 1e12
    traffic = None
    if os.path.exists(args.traffic_json):
        try:
            tj = json.load(open(args.traffic_json))
            if tj.get("kernel_source_hash") == _kernel_hash():
                traffic = tj.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None
    line = {
        "metric": "sparse prefill attn latency + effective TFLOP/s at 128K; speedup vs dense; mask density",
        "value": round(value, 2),
        "unit": "TFLOP/s (dense-equivalent causal attention FLOPs / step time)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads, "num_kv_heads": w.num_kv_heads,
                   "seq_len": L, "head_dim": d, "stride": w.stride, "block": Bk, "tau": w.tau,
                   "protect_last": True, "parallelism": "none (1 GPU)"},
        "latency_ms": round(ms_step, 4),
        "t_estimate_ms": round(t_est, 4),
        "t_sparse_attn_ms": round(t_sp, 4),
        "t_dense_attn_ms": round(t_dense, 4),
        "speedup_vs_dense": round(t_dense / ms_step, 4),
        "mask_density": round(density, 5),
        "mask_density_per_head": {"min": round(float(per_head[0]), 5),
                                  "median": round(float(per_head[len(per_head) // 2]), 5),
                                  "max": round(float(per_head[-1]), 5)},
        "mask_density_without_protected_row": round(dens_no_last, 5),
        "t_sparse_attn_ms_median_min": [round(sp_times[len(sp_times) // 2], 4), round(sp_times[0], 4)],
        "sparse_attn_unmasked_tflops": round(
            (f_sel - 4.0 * d * diag_sel * (Bk * Bk - Bk * (Bk + 1) / 2)) / (t_sp * 1e-3) / 1e12, 2),
        "estimator_kernels_ms": {kk: round(vv, 4) for kk, vv in brk.items()},
        **estimator_fracs(p, sum_cnt, t_est, brk["stride_aggregate"]),
        "dense_attn_tflops": round(f_dense / (t_dense * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "flash_attn_kernel<128,128> (rra_sparse_attn)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": f_sel, "avg_launch_ms": round(t_sp, 4)},
    }
    line["pattern_search_vs_xattn"] = pattern_search_comparison(w, qd, kd)
    ceil = mfma_ceiling()
    if ceil is not None:
        ceil["sparse_attn_frac_of_random_operand_rate"] = round(achieved / ceil["random_operands"]["tflops"], 4)
    line["mfma_sustained"] = ceil
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded sample)")
        cb = cpu_baseline(q, k, v, sel.mask.cpu().numpy(), cnt.numpy(), w, f_dense)
        line["cpu_baseline"] = {kk: (round(vv, 6) if isinstance(vv, float) else vv) for kk, vv in cb.items()}
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


def mfma_ceiling() -> dict | None:
    """Sustained bf16 MFMA rate and shader clock of a pure matrix-core loop
    (librra_probe.so), with zero and with random N(0,1) operands."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dynamic_block_sparse_sample_amd",
                        "librra_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.rra_probe_mfma_rate
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    res = {}
    for name, operands in (("zero_operands", 0), ("random_operands", 1)):
        # ~0.5 s of warm-up lets the clock settle after the attention runs (the
        # power manager reacts over tens of ms); then the median of 3 runs of ~60 ms
        runs = []
        t0 = time.time()
        while True:
            tf, ghz = ctypes.c_double(0.0), ctypes.c_double(0.0)
            rc = fn(operands, 200000, ctypes.byref(tf), ctypes.byref(ghz))
            if rc != 0:
                log(f"[bench] MFMA probe failed with HIP error {rc}")
                return None
            if time.time() - t0 > 0.5:
                runs.append((tf.value, ghz.value))
            if len(runs) == 3:
                break
        runs.sort()
        res[name] = {"tflops": round(runs[1][0], 1), "clock_ghz": round(runs[1][1], 3)}
    return res


SELECTION_POINTS = {
    "llama_8k": [(16, 0.9)],
    "llama_32k": [(s, t) for s in (8, 16, 32) for t in (0.8, 0.9, 0.95)],
    "video_64k": [(16, 0.95)],
    "llama_128k": [(16, 0.9)],
}


def estimator_fracs(p, sum_cnt: int, t_est_ms: float, t_agg_ms: float) -> dict:
    """Roofline fractions of the estimator and of its aggregation kernel.

    Algorithmic bytes of the estimator: K read once, the sampled queries, the
    mask, index lists and counts written (Kagg and block-score round trips are
    intermediates).  Binding roofline: max(bytes / BW, executed flops / P_bf16)
    / t, the two-pass scores executing 2 * 2d * Bz * H * Ns (Ns + 1) / 2 flops.
    Aggregation: K read + Kagg written over its own time."""
    L, d, nb, ns = p.seq_len, p.head_dim, p.num_blocks, p.num_strides
    k_bytes = p.batch * p.num_kv_heads * L * d * 2
    kagg_b = p.batch * p.num_kv_heads * ns * d * 2
    est_bytes = (k_bytes + p.batch * p.num_heads * ns * d * 2 + p.batch * p.num_heads * nb * nb
                 + 4 * sum_cnt + 4 * p.batch * p.num_heads * nb)
    flops2 = 2 * 2.0 * d * p.batch * p.num_heads * ns * (ns + 1) / 2
    return {
        "estimator_hbm_frac": round(est_bytes / (t_est_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "estimator_binding_roofline_frac": round(
            max(est_bytes / (PEAK_HBM_GBS * 1e9), flops2 / (PEAK_BF16_TFLOPS * 1e12)) / (t_est_ms * 1e-3), 4),
        "stride_aggregate_hbm_frac": round((k_bytes + kagg_b) / (t_agg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }


def workloads_report(reps=5):
    """Every configuration point at its own settings: the five workloads, and
    the 32K one swept over S in {8, 16, 32} x tau in {0.8, 0.9, 0.95}.  Per
    point: the estimator and its aggregation kernel, sparse and dense attention
    (event-timed averages of `reps` launches), density, TFLOP/s and roofline
    fractions.  fp32 workloads are cast to bf16 on the GPU first (timed apart)."""
    import torch

    import dynamic_block_sparse_sample_amd as rra
    from dynamic_block_sparse_sample_amd import workloads as wl

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    for name, w in wl.WORKLOADS.items():
        log(f"[workloads] {name}")
        q, k, v = wl.make_inputs(w)
        t_cast = None
        if w.fp32_inputs:
            q32, k32, v32 = q.cuda(), k.cuda(), v.cuda()
            qd, kd, vd = (torch.empty(t.shape, dtype=torch.bfloat16, device="cuda") for t in (q32, k32, v32))
            t_cast = timed(lambda: [rra.cast_f32_to_bf16(s_, d_) for s_, d_ in ((q32, qd), (k32, kd), (v32, vd))])
            del q32, k32, v32
        else:
            qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        del q, k, v
        sweep = [(S, tau) for S in (8, 16, 32) for tau in (0.8, 0.9, 0.95)] if name == "llama_32k" else [
            (w.stride, w.tau)]
        out = torch.empty_like(qd)
        t_dense = None
        for S, tau in sweep:
            p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, tau)
            ws = rra.alloc_workspace(p, qd.device)
            sel = rra.Selection(*rra._lib._selection_buffers(p, qd.device), None)
            kagg = torch.empty((p.batch, p.num_kv_heads, p.num_strides, p.head_dim), dtype=torch.bfloat16,
                               device=qd.device)
            t_est = timed(lambda: rra.estimate(p, qd, kd, workspace=ws, out=sel))
            t_agg = timed(lambda: rra.stride_aggregate(p, kd, kagg))
            t_sp = timed(lambda: rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out))
            if t_dense is None:  # depends on the shape only
                t_dense = timed(lambda: rra.dense_attn(p, qd, kd, vd, out=out))
            nb = p.num_blocks
            sum_cnt = int(sel.cnt.sum())
            f_sel = 4.0 * w.head_dim * w.block * w.block * sum_cnt
            f_full = 4.0 * w.head_dim * w.block * w.block * w.batch * w.num_heads * nb * (nb + 1) / 2
            f_dense = 4.0 * w.head_dim * w.batch * w.num_heads * w.seq_len * (w.seq_len + 1) / 2
            line = {"mode": "workloads", "workload": name, "seq_len": w.seq_len,
                    "heads": f"{w.num_heads}/{w.num_kv_heads}", "head_dim": w.head_dim, "block": w.block,
                    "stride": S, "tau": tau,
                    "density": round(sum_cnt / (w.batch * w.num_heads * nb * (nb + 1) / 2), 4),
                    "t_estimate_ms": round(t_est, 4), "t_stride_aggregate_ms": round(t_agg, 4),
                    "t_sparse_attn_ms": round(t_sp, 4), "t_dense_attn_ms": round(t_dense, 4),
                    "sparse_tflops": round(f_sel / (t_sp * 1e-3) / 1e12, 1),
                    "sparse_mfma_frac": round(f_sel / (t_sp * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "dense_tflops": round(f_full / (t_dense * 1e-3) / 1e12, 1),
                    "effective_tflops": round(f_dense / ((t_est + t_sp) * 1e-3) / 1e12, 1),
                    "speedup_vs_dense": round(t_dense / (t_est + t_sp), 3),
                    **estimator_fracs(p, sum_cnt, t_est, t_agg)}
            if t_cast is not None:
                line["t_cast_f32_to_bf16_ms"] = round(t_cast, 4)
            yield line
            del ws, sel, kagg
        del qd, kd, vd, out
        torch.cuda.empty_cache()


def xattn_supported(p) -> bool:
    """Shapes rra_xattn_block_scores is built for."""
    return (p.seq_len % p.block == 0 and p.causal == 1
            and (p.block, p.stride) in ((128, 16), (128, 8), (128, 4), (64, 8), (64, 4)))


def pattern_search_comparison(w, qd, kd, reps=5) -> dict:
    """Pattern-search time of the round-robin estimator (aggregation, scores,
    Top-tau) against XAttention's antidiagonal estimator (scores, Top-tau) on
    the same inputs, at the workload's S and at S = 8 (the pages' setting)."""
    import torch

    import dynamic_block_sparse_sample_amd as rra

    res = {}
    for S in sorted({w.stride, 8}, reverse=True):
        p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, w.tau)
        if not xattn_supported(p):
            continue
        ws = rra.alloc_workspace(p, qd.device)
        sel = rra.Selection(*rra._lib._selection_buffers(p, qd.device), None)
        score = torch.empty((p.batch, p.num_heads, p.num_blocks, p.num_blocks), dtype=torch.float32,
                            device=qd.device)
        xa_sel = rra.Selection(*rra._lib._selection_buffers(p, qd.device), None)

        def rr():
            rra.estimate(p, qd, kd, workspace=ws, out=sel)

        def xa():
            rra.xattn_block_scores(p, qd, kd, score=score)
            rra.top_tau(p, score, xa_sel.mask, xa_sel.idx, xa_sel.cnt)

        times = {}
        for name, fn in (("rr", rr), ("xattn", xa)):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            times[name] = a.elapsed_time(b) / reps
        dens = lambda c: float(c.sum()) / (p.batch * p.num_heads * p.num_blocks * (p.num_blocks + 1) / 2)  # noqa: E731
        ns = p.num_strides
        res[f"S{S}"] = {
            "rr_estimate_ms": round(times["rr"], 4), "xattn_estimate_ms": round(times["xattn"], 4),
            "rr_time_saving_vs_xattn": round(1.0 - times["rr"] / times["xattn"], 4),
            "rr_density": round(dens(sel.cnt), 5), "xattn_density": round(dens(xa_sel.cnt), 5),
            "rr_score_gflop": round(2.0 * w.head_dim * w.batch * w.num_heads * ns * (ns + 1) / 2 / 1e9, 1),
            "xattn_score_gflop": round(2.0 * S * w.head_dim * w.batch * w.num_heads * ns * (ns + 1) / 2 / 1e9, 1),
        }
    return res


def selection_report(first_workload: str):
    """Selections of the round-robin estimator (and its variants) scored
    against the exact Top-tau selection on full attention's block masses."""
    import torch

    import dynamic_block_sparse_sample_amd as rra
    from dynamic_block_sparse_sample_amd import workloads as wl
    from dynamic_block_sparse_sample_amd.selection import selection_accuracy

    names = list(SELECTION_POINTS)
    if first_workload in names and first_workload != "llama_128k":
        names = [first_workload]  # one workload when asked for a particular one
    for name in names:
        w = wl.WORKLOADS[name]
        log(f"[selection] {name}: generating inputs")
        q, k, _ = wl.make_inputs(w)
        qd, kd = q.cuda(), k.cuda()
        del q, k
        p0 = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, w.stride, w.block, w.tau)
        mass = rra.block_mass(p0, qd, kd)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        rra.block_mass(p0, qd, kd, mass=mass)
        b.record()
        torch.cuda.synchronize()
        nb = p0.num_blocks
        f_mass = 2 * 2.0 * w.head_dim * w.block * w.block * w.batch * w.num_heads * nb * (nb + 1) / 2
        t_mass = a.elapsed_time(b)
        exact = {}
        for S, tau in SELECTION_POINTS[name]:
            if tau not in exact:
                pt = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, tau)
                exact[tau] = rra.top_tau(pt, mass)[0]
            pt = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, tau)
            if rra.validate(pt) == 0 and xattn_supported(pt):
                xa_mask = rra.top_tau(pt, rra.xattn_block_scores(pt, qd, kd))[0]
                r = selection_accuracy(xa_mask, exact[tau], mass, tau)
                keys = [kk for kk in r if kk not in ("tp", "fp", "fn")]
                line = {"mode": "selection", "workload": name, "stride": S, "tau": tau, "rr": "xattn_antidiagonal",
                        "layers_averaged": 1, **{kk: round(r[kk], 5) for kk in keys},
                        "block_mass_ms": round(t_mass, 3),
                        "block_mass_tflops": round(f_mass / (t_mass * 1e-3) / 1e12, 1)}
                log(f"[selection] {name} S={S} tau={tau} xattn: F1 {r['f1']:.4f} kept {r['mass_kept_mean']:.4f}")
                yield line
            variants = [("head", [(0, 0)]), ("hybrid", [(l0, 0) for l0 in range(S)]),
                        ("layer", [(l0, 0) for l0 in range(S)]), ("none_first", [(0, 0)]),
                        ("none_last", [(0, S - 1)])]
            for label, settings in variants:
                mode = label.split("_")[0]
                acc = []
                for layer, fixed in settings:
                    p = rra.make_params(w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block,
                                        tau, rr_mode=mode, rr_layer=layer, rr_offset=fixed)
                    sel = rra.estimate(p, qd, kd)
                    acc.append(selection_accuracy(sel.mask, exact[tau], mass, tau))
                keys = [kk for kk in acc[0] if kk not in ("tp", "fp", "fn")]
                avg = {kk: round(sum(r[kk] for r in acc) / len(acc), 5) for kk in keys}
                line = {"mode": "selection", "workload": name, "stride": S, "tau": tau, "rr": label,
                        "layers_averaged": len(settings), **avg,
                        "block_mass_ms": round(t_mass, 3),
                        "block_mass_tflops": round(f_mass / (t_mass * 1e-3) / 1e12, 1)}
                log(f"[selection] {name} S={S} tau={tau} {label}: F1 {avg['f1']:.4f} "
                    f"kept {avg['mass_kept_mean']:.4f} density {avg['density_estimated']:.4f} "
                    f"(exact {avg['density_exact']:.4f})")
                yield line
        del qd, kd, mass, exact
        torch.cuda.empty_cache()


def power_report(sparse_fn, f_sparse, dense_fn, f_dense, secs) -> dict:
    """Median socket power (amd-smi, sampled from a thread) while each workload
    runs back to back, its rate, and the energy per flop above idle."""
    import ctypes
    import re
    import subprocess
    import threading

    import torch

    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                txt = subprocess.run(["amd-smi", "metric", "--power"], capture_output=True, text=True,
                                     timeout=10).stdout
                m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
                if m:
                    samples.append((time.time(), float(m.group(1))))
            except Exception:
                pass
            time.sleep(0.1)

    probe_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dynamic_block_sparse_sample_amd",
                              "librra_probe.so")
    probe = ctypes.CDLL(probe_path).rra_probe_mfma_rate
    probe.restype = ctypes.c_int
    probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    last = {}

    def mfma(operands):
        tf, ghz = ctypes.c_double(), ctypes.c_double()
        assert probe(operands, 200000, ctypes.byref(tf), ctypes.byref(ghz)) == 0
        last["tflops"], last["clock_ghz"] = tf.value, ghz.value

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    phases = []
    time.sleep(2.0)
    phases.append(("idle", time.time() - 2.0, time.time(), None, None))
    for name, fn, flops in (("sparse_attn", sparse_fn, f_sparse), ("dense_attn", dense_fn, f_dense),
                            ("mfma_probe_random_operands", lambda: mfma(1), None),
                            ("mfma_probe_zero_operands", lambda: mfma(0), None)):
        fn()
        torch.cuda.synchronize()
        t0, n = time.time(), 0
        while time.time() - t0 < secs:
            fn()
            torch.cuda.synchronize()
            n += 1
        t1 = time.time()
        rate = flops * n / (t1 - t0) / 1e12 if flops else last["tflops"]
        phases.append((name, t0, t1, rate, None if flops else last["clock_ghz"]))
        log(f"[bench] power phase {name}: {n} runs")
        time.sleep(1.5)
    stop.set()
    th.join(timeout=15)
    res = {"mode": "power", "samples": len(samples), "phases": {}}
    idle_w = None
    for name, t0, t1, rate, ghz in phases:
        v = sorted(wt for ts, wt in samples if t0 + 0.8 < ts < t1 - 0.2)
        med = v[len(v) // 2] if v else None
        if name == "idle":
            idle_w = med
        entry = {"median_w": med, "n_samples": len(v)}
        if rate is not None:
            entry["tflops"] = round(rate, 1)
            if med is not None and idle_w is not None:
                entry["pj_per_flop_above_idle"] = round((med - idle_w) / (rate * 1e12) * 1e12, 3)
        if ghz is not None:
            entry["clock_ghz"] = round(ghz, 3)
        res["phases"][name] = entry
    return res


def _kernel_hash() -> str:
    """Hash of the attention kernel source (flash_attn.hip and its work-order
    header fa_order.h); traffic counters are only valid for it."""
    import hashlib
    kdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dynamic_block_sparse_sample_amd", "csrc",
                        "kernels")
    h = hashlib.sha256()
    for name in ("flash_attn.hip", "fa_order.h"):
        with open(os.path.join(kdir, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
