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
    python bench.py --mode workloads [--cpu-oracle]   # every configuration point
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
# Exponential rate of the vector units: a wave-wide v_exp_f32 occupies its SIMD
# for 8 cycles (half the full VALU rate; measured on this chip), so 256 CUs x
# 4 SIMDs x 8 lanes per cycle x 2.4 GHz.
PEAK_EXP_T_PER_S = 256 * 4 * 8 * 2.4e9 / 1e12
COPY_BYTES = 256 << 20  # plain device copy used to calibrate the HBM byte counters
FLUSH_BYTES = 512 << 20  # written between timed repetitions to evict L2 and the 256 MB memory-side cache
FLUSH_MAX_L = 32768  # inputs of longer sequences exceed the caches by themselves
TIE_TOL = 1e-4  # near-tie rule for masks (prefix within this of tau, or masses at the cut this close)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------
class Timer:
    """Per-repetition HIP-event timing on the current stream.  Between
    repetitions, when asked, a 512 MB scratch buffer is written (outside the
    timed events) so that no input stays cached from the previous one."""

    def __init__(self, device, flush: bool):
        import torch
        self.torch = torch
        self.scratch = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=device) if flush else None

    def reps(self, fn, reps: int, warmup: int):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            if self.scratch is not None:
                self.scratch.fill_(1.0)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ev]


class ClockSampler:
    """GFX clock in MHz (mean over the XCDs) read with `amd-smi metric --clock`
    from a thread while GPU work runs; summary() keeps the samples taken inside
    a time window.  Without amd-smi it records nothing."""

    def __init__(self, period_s: float = 0.1):
        import shutil
        import threading

        self.samples = []
        self.period_s = period_s
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True) if shutil.which("amd-smi") else None

    def _read(self):
        import subprocess

        r = subprocess.run(["amd-smi", "metric", "--clock", "--json"], capture_output=True, text=True, timeout=10)
        d = json.loads(r.stdout)
        gpus = d["gpu_data"] if isinstance(d, dict) else d
        vals = []
        for name, entry in gpus[0]["clock"].items():
            clk = entry.get("clk") if isinstance(entry, dict) else None
            v = clk.get("value") if isinstance(clk, dict) else None  # "N/A" entries are strings
            if name.startswith("gfx_") and isinstance(v, (int, float)):
                vals.append(float(v))
        return sum(vals) / len(vals) if vals else None

    def _run(self):
        while not self._stop.is_set():
            t = time.time()
            try:
                v = self._read()
                if v is not None:
                    self.samples.append((t, time.time(), v))
            except Exception:
                pass
            self._stop.wait(self.period_s)

    def __enter__(self):
        if self._thread is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join(timeout=15)

    def summary(self, t0: float, t1: float):
        """Readings whose call began and ended inside [t0, t1]."""
        vals = sorted(v for ta, tb, v in self.samples if t0 <= ta and tb <= t1)
        if not vals:
            return None
        return {"samples": len(vals), "median": round(vals[len(vals) // 2], 1), "min": round(vals[0], 1),
                "max": round(vals[-1], 1)}


def clock_during(fn, secs: float):
    """GFX clock readings while fn (which synchronises) runs back to back for
    about secs seconds."""
    with ClockSampler() as cs:
        time.sleep(0.2)
        t0 = time.time()
        n = 0
        while time.time() - t0 < secs:
            fn()
            n += 1
        t1 = time.time()
    out = cs.summary(t0, t1)
    if out is not None:
        out["runs"] = n
    return out


def stats(ms):
    v = sorted(ms)
    return {"median": round(v[len(v) // 2], 4), "min": round(v[0], 4), "mean": round(sum(v) / len(v), 4),
            "n": len(v)}


# ---------------------------------------------------------------------------
# Roofline fractions
# ---------------------------------------------------------------------------
def estimator_fracs(p, sum_cnt: int, t_est_ms: float, t_agg_ms: float) -> dict:
    """Roofline fractions of the estimator and of its aggregation kernel, by
    the method's algorithmic work (single pass; the kernel's recompute is not
    counted):

      bytes = K read once + the sampled queries + mask, index lists and counts
              written (Kagg and block scores are intermediates);
      flops = 2 d Bz H Ns (Ns + 1) / 2 (each sampled query against its visible
              strides), exps = Bz H Ns (Ns + 1) / 2;
      binding fraction = max(bytes / BW, flops / P_bf16, exps / R_exp) / t.

    The two-pass kernel executes twice the flops and exps; that figure is
    reported apart.  Aggregation: K read + Kagg written over its own time."""
    L, d, nb, ns = p.seq_len, p.head_dim, p.num_blocks, p.num_strides
    k_bytes = p.batch * p.num_kv_heads * L * d * 2
    kagg_b = p.batch * p.num_kv_heads * ns * d * 2
    est_bytes = (k_bytes + p.batch * p.num_heads * ns * d * 2 + p.batch * p.num_heads * nb * nb
                 + 4 * sum_cnt + 4 * p.batch * p.num_heads * nb)
    pairs = p.batch * p.num_heads * ns * (ns + 1) / 2 if p.causal else p.batch * p.num_heads * ns * ns
    flops, exps = 2.0 * d * pairs, pairs
    floors = {"hbm": est_bytes / (PEAK_HBM_GBS * 1e9), "mfma": flops / (PEAK_BF16_TFLOPS * 1e12),
              "exp": exps / (PEAK_EXP_T_PER_S * 1e12)}
    bound = max(floors, key=floors.get)
    t = t_est_ms * 1e-3
    return {
        "estimator_algorithmic": {"bytes": est_bytes, "flops": flops, "exps": exps,
                                  "floor_us": {kk: round(vv * 1e6, 2) for kk, vv in floors.items()},
                                  "bound": bound},
        "estimator_hbm_frac": round(est_bytes / t / 1e9 / PEAK_HBM_GBS, 4),
        "estimator_binding_roofline_frac": round(floors[bound] / t, 4),
        "estimator_executed_two_pass_mfma_frac": round(2 * flops / t / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stride_aggregate_hbm_frac": round((k_bytes + kagg_b) / (t_agg_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
    }


# ---------------------------------------------------------------------------
# CPU oracle leg: timing, and the parity figures of the same calls
# ---------------------------------------------------------------------------
def _row_order(vals):
    import numpy as np
    return np.lexsort((np.arange(vals.size), -vals))


def _classify_row(gsel, osel, vals, tau):
    """'equal', 'near_tie' (differs where an oracle prefix lies within TIE_TOL
    of tau or the masses at the cut are that close) or 'other'."""
    import numpy as np
    if np.array_equal(gsel, osel):
        return "equal"
    T = vals.sum()
    if not T > 0:
        return "other"
    order = _row_order(vals)
    csum = np.cumsum(vals[order]) / T
    ks = osel.size
    prefix = np.any(np.abs(csum - tau) < TIE_TOL)
    cut = ks < vals.size and abs(vals[order[ks - 1]] - vals[order[ks]]) < TIE_TOL * vals[order[ks - 1]]
    return "near_tie" if (prefix or cut) else "other"


def _bf16_out_errors(got, ref):
    import numpy as np
    diff = np.abs(got - ref)
    _, ex = np.frexp(np.abs(ref))
    half_ulp = np.ldexp(1.0, np.maximum(ex - 1, -126) - 8)
    big = np.abs(ref) >= 1e-2
    return {"err": float(np.max(diff - half_ulp)), "max_abs": float(diff.max()),
            "max_rel": float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0}


def cpu_baseline(w, S, tau, q, k, v, gpu_mask, gpu_cnt, out, f_dense, t_gpu_ms, est_heads=None, n_rows=64,
                 full_attention=False, seed=0) -> dict:
    """The float64 CPU oracle, as it stands, on the same inputs, timed on this
    host with its BLAS limited to the cores this process may run on.

    Estimator: est_heads query heads at full length (None: every head), each
    KV group's aggregation once.  Attention: every row when full_attention,
    else n_rows seeded (head, query block) rows on the GPU's mask,
    extrapolated to the layer by selected key blocks.  Untimed, the same
    calls give the parity figures of the run: the timed heads' mask rows
    against the GPU's (equal / near-tie / other) and the attention rows'
    errors against the GPU's output (beyond half a bf16 ulp, raw max-abs, max
    relative over |exact| >= 1e-2).  q, k, v are host bf16 tensors."""
    import numpy as np
    import threadpoolctl
    from oracle import rra_oracle as orc

    cores = len(os.sched_getaffinity(0))
    H, B = w.num_heads, w.batch
    prm = orc.Params(B, H, w.num_kv_heads, w.seq_len, w.head_dim, S, w.block, float(np.float32(tau)), True)
    nb, G = prm.num_blocks, prm.group
    heads = list(range(H)) if est_heads is None else list(est_heads)
    f64 = lambda t: t.to(dtype=__import__("torch").float64).numpy()  # noqa: E731
    rows_cls = {"equal": 0, "near_tie": 0, "other": 0}
    t_est = 0.0
    t_wall0 = time.perf_counter()
    with threadpoolctl.threadpool_limits(cores):
        for b in range(B):
            kagg_g = None
            for h in heads:
                g = h // G
                if kagg_g is None or kagg_g[0] != g:
                    kg = f64(k[b, g])
                    t0 = time.perf_counter()
                    kagg_g = (g, orc.aggregate_keys(kg, S))
                    t_est += time.perf_counter() - t0
                qh = f64(q[b, h])
                t0 = time.perf_counter()
                s = orc.stride_scores(qh, kagg_g[1], S, h, prm.scale)
                m = orc.pool_blocks(orc.stride_softmax(s), prm.strides_per_block)
                sels = [orc.top_tau_row(m[i], i, prm.tau, i == nb - 1) for i in range(nb)]
                t_est += time.perf_counter() - t0
                for i in range(nb):
                    gsel = np.nonzero(gpu_mask[b, h, i, :i + 1])[0]
                    rows_cls[_classify_row(gsel, sels[i], m[i, :i + 1], prm.tau)] += 1
        t_est_layer = t_est * (H / len(heads))
        if full_attention:
            rows = [(b, h, i) for b in range(B) for h in range(H) for i in range(nb)]
        else:
            rng = np.random.default_rng(seed)
            rows = sorted({(int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(nb)))
                           for _ in range(4 * n_rows)})
            rng.shuffle(rows)
            rows = sorted(rows[:n_rows])
        one = orc.Params(1, 1, 1, prm.seq_len, prm.head_dim, S, prm.block, prm.tau, True)
        t_attn, blocks, errs, cur = 0.0, 0, None, None
        for (b, h, i) in rows:
            if cur != (b, h):
                cur = (b, h)
                g = h // G
                qh, kh, vh = f64(q[b:b + 1, h:h + 1]), f64(k[b:b + 1, g:g + 1]), f64(v[b:b + 1, g:g + 1])
                mh = gpu_mask[b:b + 1, h:h + 1]
            t0 = time.perf_counter()
            ref = orc.attention_rows(qh, kh, vh, mh, one, 0, 0, i)
            t_attn += time.perf_counter() - t0
            blocks += int(gpu_cnt[b, h, i])
            got = f64(out[b, h, i * prm.block:i * prm.block + ref.shape[0]].cpu())
            e = _bf16_out_errors(got, ref)
            errs = e if errs is None else {kk: max(errs[kk], e[kk]) for kk in e}
        t_attn_layer = t_attn if full_attention else t_attn / max(blocks, 1) * float(gpu_cnt.sum())
    t_total = t_est_layer + t_attn_layer
    extrapolated = est_heads is not None or not full_attention
    return {
        "value": f_dense / t_total / 1e12,
        "unit": "TFLOP/s (dense-equivalent causal attention FLOPs / oracle step time)",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle, BLAS limited to {cores} threads (elementwise steps single-threaded): "
                   f"estimator on {len(heads)} of {H} heads at full length ({t_est:.1f} s), attention on "
                   + ("every row" if full_attention else f"{len(rows)} seeded (head, query block) rows")
                   + f" ({blocks} key blocks, {t_attn:.1f} s)"
                   + ("; extrapolated to the layer by heads and by selected key blocks" if extrapolated else "")
                   + f": {t_total:.1f} s per step"),
        "extrapolated": extrapolated,
        "s_per_step": t_total,
        "estimate_s": t_est_layer,
        "sparse_attn_s": t_attn_layer,
        "gpu_over_cpu": t_total / (t_gpu_ms * 1e-3),
        "wall_s": time.perf_counter() - t_wall0,
        "cpu_model": _cpu_model(),
        "parity": {"mask_rows_compared": sum(rows_cls.values()), **{f"mask_rows_{kk}": vv for kk, vv in
                                                                   rows_cls.items()},
                   "output_rows_compared": len(rows), "output_err_beyond_half_ulp": errs["err"],
                   "output_max_abs": errs["max_abs"], "output_max_rel": errs["max_rel"]},
    }


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _round_floats(d):
    if isinstance(d, dict):
        return {kk: _round_floats(vv) for kk, vv in d.items()}
    if isinstance(d, float):
        return float(f"{d:.6g}")
    return d


# ---------------------------------------------------------------------------
# Headline step
# ---------------------------------------------------------------------------
def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama_128k")
    ap.add_argument("--dense-reps", type=int, default=3)
    ap.add_argument("--reps", type=int, default=20, help="timed repetitions per point (workloads mode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-oracle", action="store_true",
                    help="workloads mode: also time the CPU oracle per point (estimator over every head; "
                         "attention in full at 1K and 8K, else 64 seeded rows) with its parity figures")
    ap.add_argument("--mode", choices=["bench", "profile", "power", "selection", "workloads"], default="bench",
                    help="profile: one estimate, --steps sparse-attention launches, one dense launch and a "
                         "256 MiB device copy (HBM-counter calibration); prints a short summary only. "
                         "power: socket power (amd-smi) while sparse and dense attention each run back to "
                         "back for --power-secs seconds. "
                         "selection: precision / recall / F1 and kept attention mass of the estimated "
                         "selections (round-robin variants, several S and tau) against the exact Top-tau "
                         "selection, one JSON line per point. workloads: estimate / sparse / dense times "
                         "(median and min of --reps, caches flushed between repetitions up to 32K) and "
                         "density of every workload at its own settings, one JSON line each")
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
        for line in workloads_report(args.reps, args.cpu_oracle):
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
    sp_times = [a.elapsed_time(b) for a, b in sp_ev]
    est_times = [a.elapsed_time(b) for a, b in est_ev]
    t_sp = sum(sp_times) / args.steps
    t_est = sum(est_times) / args.steps
    log(f"[bench] {ms_step:.3f} ms per step (estimate {t_est:.3f}, sparse attention {t_sp:.3f})")

    # per-kernel breakdown of the estimator (same buffers)
    kagg = ws[: p.batch * p.num_kv_heads * p.num_strides * p.head_dim * 2].view(torch.bfloat16).view(
        p.batch, p.num_kv_heads, p.num_strides, p.head_dim)
    score = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=dev)
    timer = Timer(dev, flush=w.seq_len <= FLUSH_MAX_L)
    brk = {}
    for name, fn in [("stride_aggregate", lambda: rra.stride_aggregate(p, kd, kagg)),
                     ("block_scores", lambda: rra.block_scores(p, qd, kagg, score)),
                     ("top_tau", lambda: rra.top_tau(p, score, sel.mask, sel.idx, sel.cnt))]:
        brk[name] = stats(timer.reps(fn, 5, 1))
    del score

    log(f"[bench] dense baseline x{args.dense_reps}")
    dn_times = timer.reps(lambda: rra.dense_attn(p, qd, kd, vd, out=dense_out), args.dense_reps, 1)
    t_dense = sum(dn_times) / len(dn_times)

    # the timed steps left the selection and output of this input in sel / out
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
        "t_estimate_ms_stats": stats(est_times),
        "t_sparse_attn_ms_stats": stats(sp_times),
        "t_dense_attn_ms_stats": stats(dn_times),
        "speedup_vs_dense": round(t_dense / ms_step, 4),
        "mask_density": round(density, 5),
        "mask_density_per_head": {"min": round(float(per_head[0]), 5),
                                  "median": round(float(per_head[len(per_head) // 2]), 5),
                                  "max": round(float(per_head[-1]), 5)},
        "mask_density_without_protected_row": round(dens_no_last, 5),
        "sparse_attn_unmasked_tflops": round(
            (f_sel - 4.0 * d * diag_sel * (Bk * Bk - Bk * (Bk + 1) / 2)) / (t_sp * 1e-3) / 1e12, 2),
        "estimator_kernels_ms": brk,
        **estimator_fracs(p, sum_cnt, t_est, brk["stride_aggregate"]["median"]),
        "dense_attn_tflops": round(f_dense / (t_dense * 1e-3) / 1e12, 2),
        # GFX clock (amd-smi, mean over the XCDs), read after the timed region while the step and the
        # dense launch each run back to back for a few seconds
        "gpu_clock_mhz": {"step": clock_during(lambda: (step(), torch.cuda.synchronize()), 4.0),
                          "dense_attn": clock_during(lambda: (rra.dense_attn(p, qd, kd, vd, out=dense_out),
                                                              torch.cuda.synchronize()), 4.0)},
        "roofline": {"kernel": "flash_attn_kernel<128,128> (rra_sparse_attn)", "bound": "mfma",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "flops_per_launch": f_sel, "avg_launch_ms": round(t_sp, 4)},
    }
    line["pattern_search_vs_xattn"] = pattern_search_comparison(w, qd, kd)
    if not args.no_cpu_baseline:
        log("[bench] CPU oracle baseline (bounded sample: 4 heads' estimator, 64 attention rows)")
        cb = cpu_baseline(w, w.stride, w.tau, q, k, v, sel.mask.cpu().numpy(), cnt.numpy(), out, f_dense, ms_step,
                          est_heads=[0, 9, 18, 27] if w.num_heads >= 28 else None, n_rows=64, seed=0)
        line["cpu_baseline"] = _round_floats(cb)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


# ---------------------------------------------------------------------------
# Every configuration point
# ---------------------------------------------------------------------------
def workloads_report(reps=20, cpu_oracle=False):
    """Every configuration point at its own settings: the five workloads, and
    the 32K one swept over S in {8, 16, 32} x tau in {0.8, 0.9, 0.95}.  Per
    point: the estimator and its aggregation kernel, sparse and dense attention
    (median and min of `reps` event-timed launches after 5 warm-ups, a 512 MB
    scratch write between launches up to 32K), density, TFLOP/s and roofline
    fractions; with cpu_oracle, the CPU oracle's time for the point and its
    parity figures.  fp32 workloads are cast to bf16 on the GPU first (timed
    apart)."""
    import torch

    import dynamic_block_sparse_sample_amd as rra
    from dynamic_block_sparse_sample_amd import workloads as wl

    for name, w in wl.WORKLOADS.items():
        log(f"[workloads] {name}")
        q, k, v = wl.make_inputs(w)
        timer = Timer("cuda", flush=w.seq_len <= FLUSH_MAX_L)
        t_cast = None
        if w.fp32_inputs:
            q32, k32, v32 = q.cuda(), k.cuda(), v.cuda()
            qd, kd, vd = (torch.empty(t.shape, dtype=torch.bfloat16, device="cuda") for t in (q32, k32, v32))
            t_cast = stats(timer.reps(lambda: [rra.cast_f32_to_bf16(s_, d_) for s_, d_ in
                                               ((q32, qd), (k32, kd), (v32, vd))], reps, 5))
            del q32, k32, v32
            q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))  # what the GPU computes on (RNE, as the cast)
        else:
            qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
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
            t_est = stats(timer.reps(lambda: rra.estimate(p, qd, kd, workspace=ws, out=sel), reps, 5))
            t_agg = stats(timer.reps(lambda: rra.stride_aggregate(p, kd, kagg), reps, 5))
            t_sp = stats(timer.reps(lambda: rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out), reps, 5))
            if t_dense is None:  # depends on the shape only
                t_dense = stats(timer.reps(lambda: rra.dense_attn(p, qd, kd, vd, out=out), max(reps // 2, 3), 2))
            rra.sparse_attn(p, qd, kd, vd, sel.idx, sel.cnt, out=out)
            torch.cuda.synchronize()
            nb = p.num_blocks
            sum_cnt = int(sel.cnt.sum())
            f_sel = 4.0 * w.head_dim * w.block * w.block * sum_cnt
            f_full = 4.0 * w.head_dim * w.block * w.block * w.batch * w.num_heads * nb * (nb + 1) / 2
            f_dense = 4.0 * w.head_dim * w.batch * w.num_heads * w.seq_len * (w.seq_len + 1) / 2
            te, ts, td = t_est["median"], t_sp["median"], t_dense["median"]
            line = {"mode": "workloads", "workload": name, "seq_len": w.seq_len,
                    "heads": f"{w.num_heads}/{w.num_kv_heads}", "head_dim": w.head_dim, "block": w.block,
                    "stride": S, "tau": tau, "caches_flushed": timer.scratch is not None,
                    "density": round(sum_cnt / (w.batch * w.num_heads * nb * (nb + 1) / 2), 4),
                    "t_estimate_ms": t_est, "t_stride_aggregate_ms": t_agg,
                    "t_sparse_attn_ms": t_sp, "t_dense_attn_ms": t_dense,
                    "sparse_tflops": round(f_sel / (ts * 1e-3) / 1e12, 1),
                    "sparse_mfma_frac": round(f_sel / (ts * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "dense_tflops": round(f_full / (td * 1e-3) / 1e12, 1),
                    "effective_tflops": round(f_dense / ((te + ts) * 1e-3) / 1e12, 1),
                    "speedup_vs_dense": round(td / (te + ts), 3),
                    **estimator_fracs(p, sum_cnt, te, t_agg["median"])}
            if t_cast is not None:
                line["t_cast_f32_to_bf16_ms"] = t_cast
            if cpu_oracle:
                log(f"[workloads] {name} S={S} tau={tau}: CPU oracle")
                full_attn = w.seq_len <= 8192
                cb = cpu_baseline(w, S, tau, q, k, v, sel.mask.cpu().numpy(), sel.cnt.cpu().numpy(), out,
                                  f_dense, te + ts, est_heads=None, n_rows=64, full_attention=full_attn, seed=S)
                line["cpu_oracle"] = _round_floats(cb)
            log(f"[workloads] {name} S={S} tau={tau}: sparse {ts:.3f} ms, dense {td:.3f} ms, "
                f"estimate {te:.3f} ms, density {line['density']}")
            yield line
            del ws, sel, kagg
        del qd, kd, vd, out, timer
        torch.cuda.empty_cache()


def power_report(sparse_fn, f_sparse, dense_fn, f_dense, secs) -> dict:
    """Median socket power (amd-smi, sampled from a thread) while each workload
    runs back to back, its rate, and the energy per flop above idle."""
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

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    phases = []
    with ClockSampler(period_s=0.2) as clocks:
        time.sleep(2.0)
        phases.append(("idle", time.time() - 2.0, time.time(), None))
        for name, fn, flops in (("sparse_attn", sparse_fn, f_sparse), ("dense_attn", dense_fn, f_dense)):
            fn()
            torch.cuda.synchronize()
            t0, n = time.time(), 0
            while time.time() - t0 < secs:
                fn()
                torch.cuda.synchronize()
                n += 1
            t1 = time.time()
            phases.append((name, t0, t1, flops * n / (t1 - t0) / 1e12))
            log(f"[bench] power phase {name}: {n} runs")
            time.sleep(1.5)
    stop.set()
    th.join(timeout=15)
    res = {"mode": "power", "samples": len(samples), "phases": {}}
    idle_w = None
    for name, t0, t1, rate in phases:
        vals = sorted(wt for ts, wt in samples if t0 + 0.8 < ts < t1 - 0.2)
        med = vals[len(vals) // 2] if vals else None
        if name == "idle":
            idle_w = med
        entry = {"median_w": med, "n_samples": len(vals), "gfx_clock_mhz": clocks.summary(t0 + 0.8, t1 - 0.2)}
        if rate is not None:
            entry["tflops"] = round(rate, 1)
            if med is not None and idle_w is not None:
                entry["pj_per_flop_above_idle"] = round((med - idle_w) / (rate * 1e12) * 1e12, 3)
        res["phases"][name] = entry
    return res


SELECTION_POINTS = {
    "llama_8k": [(16, 0.9)],
    "llama_32k": [(s, t) for s in (8, 16, 32) for t in (0.8, 0.9, 0.95)],
    "video_64k": [(16, 0.95)],
    "llama_128k": [(16, 0.9)],
}


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


def _kernel_hash() -> str:
    """Hash of the attention kernel source (flash_attn.hip and the headers of
    its directory that it includes: the work order, the LDS copies and the
    device helpers); traffic counters are only valid for it."""
    import hashlib
    kdir = os.path.join(os.path.dirname(os.path.abspath(__file__)), "dynamic_block_sparse_sample_amd", "csrc",
                        "kernels")
    h = hashlib.sha256()
    for name in ("flash_attn.hip", "fa_order.h", "lds_copy.h", "rra_device.h"):
        with open(os.path.join(kdir, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]



if __name__ == "__main__":
    sys.exit(main())
