"""Mutation check of the oracle's pins (run by hand, on the CPU):

    python tests/oracle_mutants.py [name-substring ...]

Each mutant plants one plausible mistake in a temporary copy of
oracle/rra_oracle.py (a dropped term, a wrong index, axis, comparison or
rounding mode, a swapped head mapping) and runs the CPU suite
(pytest -m "not gpu") on that copy.  Every mutant must be killed: some CPU
test fails.  Exit status 1 if any survives or its pattern is gone.
"""
import os
import shutil
import subprocess
import sys
import tempfile

SRC = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTANTS = [
    ("agg: no 1/S", "    mean = sums / stride\n", "    mean = sums\n"),
    ("agg: 1/(S-1)", "    mean = sums / stride\n", "    mean = sums / max(stride - 1, 1)\n"),
    ("scores: no rr offset", "s[have] = sm_scale * (q_head[pos[have]] @ kagg.T)", "s[have] = sm_scale * (q_head[(np.arange(ns) * stride)[have]] @ kagg.T)"),
    ("scores: diagonal stride masked", "upper = np.triu(np.ones((ns, ns), dtype=bool), k=1) & have[:, None]", "upper = np.triu(np.ones((ns, ns), dtype=bool), k=0) & have[:, None]"),
    ("scores: no sm_scale", "s[have] = sm_scale * (q_head[pos[have]] @ kagg.T)", "s[have] = (q_head[pos[have]] @ kagg.T)"),
    ("softmax: global normalisation", "out[ok] = e / np.sum(e, axis=1, keepdims=True)", "out[ok] = e / np.sum(e)"),
    ("softmax: column axis", "    m = np.max(s[ok], axis=1, keepdims=True)\n    e = np.exp(s[ok] - m)\n    out[ok] = e / np.sum(e, axis=1, keepdims=True)", "    m = np.max(s[ok], axis=1, keepdims=True)\n    e = np.exp(s[ok] - m)\n    out[ok] = e / np.maximum(np.sum(e, axis=0, keepdims=True), 1e-300)"),
    ("pool: divide by r always", "return np.where(count[:, None] > 0, sums / np.maximum(count, 1)[:, None], 0.0)", "return np.where(count[:, None] > 0, sums / r, 0.0)"),
    ("pool: transposed", "sums = pp.reshape(nb, r, nb, r).sum(axis=(1, 3))", "sums = pp.reshape(nb, r, nb, r).sum(axis=(1, 3)).T"),
    ("pool: no mean (sum)", "return np.where(count[:, None] > 0, sums / np.maximum(count, 1)[:, None], 0.0)", "return np.where(count[:, None] > 0, sums, 0.0)"),
    ("top_tau: > instead of >=", "hit = np.nonzero(csum >= tau * total)[0]", "hit = np.nonzero(csum > tau * total)[0]"),
    ("top_tau: ties J desc", "order = np.lexsort((np.arange(n), -vals))", "order = np.lexsort((-np.arange(n), -vals))"),
    ("top_tau: one block too many", "k_star = int(hit[0]) + 1 if hit.size else n", "k_star = min(int(hit[0]) + 2, n) if hit.size else n"),
    ("top_tau: protection ignored", "    if tau >= 1.0 or protect:\n", "    if tau >= 1.0:\n"),
    ("select: protect first row", "prm.protect_last and i == nb - 1", "prm.protect_last and i == 0"),
    ("attend: causal off by one", "        s[key_pos[None, :] > q_pos[:, None]] = -np.inf\n    m = np.max", "        s[key_pos[None, :] >= q_pos[:, None] + 1 - 1 + (q_pos[:, None] > 0)] = -np.inf\n    m = np.max"),
    ("attend: no causal mask", "    if causal:\n        s[key_pos[None, :] > q_pos[:, None]] = -np.inf\n    m = np.max", "    if False:\n        s[key_pos[None, :] > q_pos[:, None]] = -np.inf\n    m = np.max"),
    ("mass: mean over Bk", "out[:nbk] = pp.reshape(t.size, nbk, bk).sum(axis=(0, 2)) / t.size", "out[:nbk] = pp.reshape(t.size, nbk, bk).sum(axis=(0, 2)) / bk"),
    ("mass: diagonal key excluded", "        s[np.arange(n_keys)[None, :] > t[:, None]] = -np.inf\n    e = np.exp", "        s[np.arange(n_keys)[None, :] >= t[:, None]] = -np.inf\n        s[:, 0] = np.where(t == 0, 0.0, s[:, 0])\n    e = np.exp"),
    ("bf16: truncation", "    r = np.rint(x[nz] / ulp) * ulp\n", "    r = np.trunc(x[nz] / ulp) * ulp\n"),
    ("bf16: ties away", "    r = np.rint(x[nz] / ulp) * ulp\n", "    r = np.sign(x[nz]) * np.floor(np.abs(x[nz]) / ulp + 0.5) * ulp\n"),
    ("rr: hybrid = head", "        return (head + layer) % stride\n", "        return head % stride\n"),
    ("rr: head+1", "    if mode == \"head\":\n        return head % stride\n", "    if mode == \"head\":\n        return (head + 1) % stride\n"),
    ("xattn: queries not reversed", "qrev = q[b, h].reshape(ns, S, d)[:, ::-1, :].reshape(ns, S * d)", "qrev = q[b, h].reshape(ns, S, d).reshape(ns, S * d)"),
    ("gqa: wrong kv head", "            kagg = aggregate_keys(k[b, g], prm.stride, kagg_round)\n", "            kagg = aggregate_keys(k[b, (g + 1) % prm.num_kv_heads], prm.stride, kagg_round)\n"),
    ("attn: gqa group", "    g = h // prm.group\n", "    g = h % prm.num_kv_heads\n"),
]

def main() -> int:
    only = sys.argv[1:]
    with open(os.path.join(SRC, "oracle", "rra_oracle.py")) as f:
        orig = f.read()
    bad = 0
    with tempfile.TemporaryDirectory() as tmp:
        dst = os.path.join(tmp, "repo")
        os.makedirs(dst)
        skip = shutil.ignore_patterns("*.so", "*.o", "__pycache__")
        for name in ("oracle", "tests", "dynamic_block_sparse_sample_amd", "include"):
            shutil.copytree(os.path.join(SRC, name), os.path.join(dst, name), ignore=skip)
        for name in ("pytest.ini", "bench.py", "__graft_entry__.py"):
            shutil.copy2(os.path.join(SRC, name), dst)
        target = os.path.join(dst, "oracle", "rra_oracle.py")
        for name, a, b in MUTANTS:
            if only and not any(o in name for o in only):
                continue
            if a not in orig:
                print(f"{name:34s} PATTERN NOT FOUND", flush=True)
                bad += 1
                continue
            with open(target, "w") as f:
                f.write(orig.replace(a, b, 1))
            r = subprocess.run([sys.executable, "-m", "pytest", "tests", "-q", "-x", "-m", "not gpu",
                                "-p", "no:cacheprovider"], cwd=dst, capture_output=True, text=True, timeout=900)
            lines = [line for line in r.stdout.splitlines() if line.strip()]
            last = lines[-1] if lines else r.stderr[-200:]
            killed = r.returncode != 0
            bad += 0 if killed else 1
            print(f"{name:34s} {'killed' if killed else 'SURVIVED'}: {last[:100]}", flush=True)
    return 1 if bad else 0


if __name__ == "__main__":
    sys.exit(main())
