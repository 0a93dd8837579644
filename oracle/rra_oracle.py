"""Plain, slow CPU oracle for RRAttention block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and the
CPU-baseline leg of the benchmark may import this module. The library's
product path never calls it, and this module imports nothing from the HIP path.

Everything is computed in float64 with numpy, head by head, in the order the
method is described in

    "RRAttention: Dynamic Block Sparse Attention via Per-Head Round-Robin
    Shifts for Long-Context Inference" (arXiv 2602.05853):
      §2.1 Block-wise Sparse Attention        -- block partition, stride S
      §3.1 Query Sampling with Head Round-Robin Strategy
      §3.2 Stride-level Importance Estimation -- stride scores, 1/(S*sqrt(d))
      §3.3 Block-level Selection via Top-tau Thresholding
      §4.1 Settings                           -- prefill only, FlashAttention baseline
      §4.3 Ablation Study                     -- last-query-block protection
      §7   Limitations                        -- S > H coverage gap
    and the XAttention summary page (arXiv 2503.16428), "Key points": keep the
    minimal set of blocks whose cumulative normalised score reaches tau.

Several displayed equations of the RRAttention page were lost (the sampling
formula of §3.1, the score equation of §3.2, all of §3.3).  The readings used
here are:

  * sampled position  P(i, h) = i*S + (h mod S)                    (§3.1, §7)
  * round-robin variants of the §4.3 ablation (named there, not defined):
                      layer-RR  o = l mod S, hybrid-RR  o = (h + l) mod S,
                      no RR  o = a fixed offset c, with P(i, h) = i*S + o
  * aggregated key    Kagg[j] = bf16_rne( (sum of K over stride j) / S )
                      -- the 1/S of the §3.2 normalisation folded into the
                      stride mean; the bf16 rounding is part of the library's
                      contract ("none" skips it)
  * stride score      s[i, j] = sm_scale * <Q[P(i,h)], Kagg[j]>,  j <= i
  * stride softmax    per sampled query, over its visible strides (§2.2 query
                      independence)
  * block score       M[I, J] = (1/r) * sum_{i in I} sum_{j in J, j <= i} p[i, j],
                      r = Bk / S, so every row of M sums to 1
  * Top-tau           order J by (M desc, J asc); keep the first k* with
                      cumulative mass >= tau * (row total); tau >= 1 or the
                      protected last query-block row keeps all causal blocks
  * attention         exact causal softmax attention restricted, per query,
                      to keys in its selected key blocks

Indices are 0-based.  GQA: query head h reads KV head h // (H / Hkv).

Parity status: every function below is pinned by a CPU test against a closed
form, a library routine, brute force or a hand-worked table.  Faithfulness of
the readings above to the authors' own (unpublished) implementation is parity
unpinned: the pages print no worked example.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Params",
    "bf16_round",
    "rr_offset",
    "rr_positions",
    "aggregate_keys",
    "stride_scores",
    "stride_softmax",
    "pool_blocks",
    "block_scores",
    "top_tau_row",
    "select_blocks",
    "estimate",
    "exact_block_mass",
    "xattn_block_scores",
    "exact_block_mass_row",
    "block_sparse_attention",
    "dense_attention",
    "attention_rows",
]


@dataclass(frozen=True)
class Params:
    """Problem sizes and sparsity settings (RRAttention §2.1, §4.1)."""

    batch: int
    num_heads: int
    num_kv_heads: int
    seq_len: int
    head_dim: int
    stride: int  # S
    block: int  # Bk (the page calls it B)
    tau: float
    protect_last: bool = True
    sm_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)
    rr_mode: str = "head"  # "head", "layer", "hybrid" or "none" (§4.3 ablation)
    rr_layer: int = 0  # layer index l for "layer" and "hybrid"
    rr_fixed: int = 0  # the offset for "none"
    causal: bool = True  # False: every key visible to every query (encoder / generation use)

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def num_strides(self) -> int:
        return -(-self.seq_len // self.stride)  # ceil: a last partial stride counts

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block)  # ceil(L / B), §2.1

    @property
    def strides_per_block(self) -> int:
        return self.block // self.stride


# ---------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), from the definition.
# ---------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (7 stored) and float32's exponent
    range.  For |x| in [2^e, 2^(e+1)) the spacing of bf16 values is
    2^(e-7); below 2^-126 (bf16 subnormals) the spacing is fixed at 2^-133.
    Dividing by a power of two is exact in float64, and numpy's rint rounds
    half to even, so x / ulp -> rint -> * ulp is the exact RNE result.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, ex = np.frexp(x[nz])  # x = m * 2^ex, 0.5 <= |m| < 1  ->  e = ex - 1
    e = np.maximum(ex - 1, -126)
    ulp = np.ldexp(1.0, e - 7)
    r = np.rint(x[nz] / ulp) * ulp
    if np.any(np.abs(r) >= 2.0**128):
        raise OverflowError("value outside the bfloat16 finite range")
    out[nz] = r
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


# ---------------------------------------------------------------------------
# §3.1: head round-robin query sampling.
# ---------------------------------------------------------------------------
def rr_offset(head: int, stride: int, mode: str = "head", layer: int = 0, fixed: int = 0) -> int:
    """Offset inside every stride of the query sampled for `head`.

    head-RR (the method, §3.1): the offset rotates with the head index.  The
    §4.3 ablation also names layer-RR, hybrid-RR and no RR without formulas;
    read as rotating with the layer index, with head plus layer, and not at
    all (one fixed offset for every head and layer).
    """
    if mode == "head":
        return head % stride
    if mode == "layer":
        return layer % stride
    if mode == "hybrid":
        return (head + layer) % stride
    if mode == "none":
        if not 0 <= fixed < stride:
            raise ValueError("fixed offset outside the stride")
        return fixed
    raise ValueError(f"unknown round-robin mode {mode!r}")


def rr_positions(num_strides: int, stride: int, head: int, mode: str = "head", layer: int = 0,
                 fixed: int = 0) -> np.ndarray:
    """Token position sampled from each stride i for query head `head`.

    One query per stride of S tokens; the offset inside the stride rotates
    with the head index (RRAttention §1, §3.1 and the abstract) and does not
    depend on i, so with S > H some offsets are never sampled (§7).
    """
    return np.arange(num_strides, dtype=np.int64) * stride + rr_offset(head, stride, mode, layer, fixed)


# ---------------------------------------------------------------------------
# §3.2: stride-level key aggregation and scores.
# ---------------------------------------------------------------------------
def aggregate_keys(k_head: np.ndarray, stride: int, kagg_round: str = "bf16") -> np.ndarray:
    """Mean of the S key vectors of every stride j, for one KV head.

    k_head: [L, d] float64 holding bf16 values.  The sum of S <= 32 bf16
    values is exact in float64 (it needs far fewer than 53 bits for any data
    whose magnitudes span under 2^40), and /S is exact for a power-of-two S.
    """
    L, d = k_head.shape
    ns = -(-L // stride)
    padded = np.zeros((ns * stride, d))
    padded[:L] = k_head  # a last partial stride sums the keys it has; the 1/S stays
    sums = padded.reshape(ns, stride, d).sum(axis=1)
    mean = sums / stride
    if kagg_round == "bf16":
        return bf16_round(mean)
    if kagg_round == "none":
        return mean
    raise ValueError(f"unknown kagg_round {kagg_round!r}")


def stride_scores(q_head: np.ndarray, kagg: np.ndarray, stride: int, head: int,
                  sm_scale: float, mode: str = "head", layer: int = 0, fixed: int = 0,
                  causal: bool = True) -> np.ndarray:
    """s[i, j] = sm_scale * <Q[P(i, h)], Kagg[j]> for j <= i, -inf above.

    With Kagg the stride mean, sm_scale = 1/sqrt(d) gives the page's
    normalisation 1/(S*sqrt(d)) of Q_P(i,h) . sum_{t in stride j} K_t.
    Every stride j <= i is visible, the diagonal stride included; every
    stride when not causal.  Rows whose sampled position lies beyond the
    sequence (a last partial stride) are NaN: that stride has no query.
    """
    ns = kagg.shape[0]
    pos = rr_positions(ns, stride, head, mode, layer, fixed)
    have = pos < q_head.shape[0]  # a last partial stride may hold no sampled query: NaN row
    s = np.full((ns, ns), np.nan)
    s[have] = sm_scale * (q_head[pos[have]] @ kagg.T)
    if causal:
        upper = np.triu(np.ones((ns, ns), dtype=bool), k=1) & have[:, None]
        s[upper] = -np.inf
    return s


def stride_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax of every sampled query's row over its visible strides (§2.2).
    Rows without a query (NaN) stay NaN."""
    out = np.full(s.shape, np.nan)
    ok = ~np.isnan(s).any(axis=1)
    m = np.max(s[ok], axis=1, keepdims=True)
    e = np.exp(s[ok] - m)
    out[ok] = e / np.sum(e, axis=1, keepdims=True)
    return out


def pool_blocks(p: np.ndarray, strides_per_block: int) -> np.ndarray:
    """M[I, J] = (1/r_I) * sum of p over the stride cells of block (I, J).

    r_I is the number of sampled queries block I holds: r = Bk / S for a
    whole block, fewer for a last partial block; each row sums to 1.  A block
    without any sampled query gets a zero row (no estimate).
    """
    ns = p.shape[0]
    r = strides_per_block
    nb = -(-ns // r)
    rows = ~np.isnan(p).any(axis=1)
    pp = np.zeros((nb * r, nb * r))
    pp[:ns, :ns][rows] = p[rows]
    count = np.zeros(nb * r)
    count[:ns] = rows
    count = count.reshape(nb, r).sum(axis=1)
    sums = pp.reshape(nb, r, nb, r).sum(axis=(1, 3))
    return np.where(count[:, None] > 0, sums / np.maximum(count, 1)[:, None], 0.0)


def block_scores(q: np.ndarray, k: np.ndarray, prm: Params, kagg_round: str = "bf16") -> np.ndarray:
    """Block-score matrices M for every (batch, query head): [Bz, H, Nb, Nb]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    nb = prm.num_blocks
    out = np.zeros((prm.batch, prm.num_heads, nb, nb))
    for b in range(prm.batch):
        for g in range(prm.num_kv_heads):
            kagg = aggregate_keys(k[b, g], prm.stride, kagg_round)
            for hh in range(prm.group):
                h = g * prm.group + hh
                s = stride_scores(q[b, h], kagg, prm.stride, h, prm.scale, prm.rr_mode, prm.rr_layer,
                                  prm.rr_fixed, prm.causal)
                out[b, h] = pool_blocks(stride_softmax(s), prm.strides_per_block)
    return out


def xattn_block_scores(q: np.ndarray, k: np.ndarray, prm: Params) -> np.ndarray:
    """XAttention's antidiagonal block scores, for comparison: [Bz, H, Nb, Nb].

    Inside each S x S cell (query stride i, key stride j) of the token score
    matrix, the entries on the antidiagonal running from the lower left to the
    upper right are summed (XA summary and key points; RR §2.2 describes it as
    aggregation across different queries).  With the queries of stride i
    concatenated in reverse order and the keys of stride j concatenated in
    order, that sum is one dot product of length S*d.  Normalised by
    1/(S*sqrt(d)) like RR §3.2's stride scores, softmax per query stride over
    the key strides j <= i, pooled into blocks with 1/r exactly as
    block_scores does.  Whole blocks and causal attention only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    S, ns, nb, d = prm.stride, prm.num_strides, prm.num_blocks, prm.head_dim
    if prm.seq_len % prm.block or not prm.causal:
        raise ValueError("xattn_block_scores: whole blocks and causal attention only")
    out = np.zeros((prm.batch, prm.num_heads, nb, nb))
    for b in range(prm.batch):
        for h in range(prm.num_heads):
            qrev = q[b, h].reshape(ns, S, d)[:, ::-1, :].reshape(ns, S * d)
            kcat = k[b, h // prm.group].reshape(ns, S * d)
            a = (prm.scale / S) * (qrev @ kcat.T)
            a[np.triu_indices(ns, k=1)] = -np.inf
            out[b, h] = pool_blocks(stride_softmax(a), prm.strides_per_block)
    return out


def exact_block_mass(q: np.ndarray, k: np.ndarray, prm: Params) -> np.ndarray:
    """Block masses of full causal softmax attention: [Bz, H, Nb, Nb].

    M*[I, J] = (1/Bk) * sum_{t in I} sum_{u in J, u <= t} p[t, u], with p the
    causal softmax of sm_scale * q_t . k_u over u <= t (over every key when
    not causal; a last partial block averages over the queries it has).  This is what the
    estimator's block score stands for (§3.2 with every query sampled and no
    key aggregation); Top-tau on it (§3.3) is the exact selection the sampled
    one is scored against.
    """
    nb = prm.num_blocks
    out = np.zeros((prm.batch, prm.num_heads, nb, nb))
    for b in range(prm.batch):
        for h in range(prm.num_heads):
            for i in range(nb):
                out[b, h, i] = exact_block_mass_row(q, k, prm, b, h, i)
    return out


def exact_block_mass_row(q, k, prm: Params, b: int, h: int, row: int) -> np.ndarray:
    """Row `row` of exact_block_mass for (b, h): [Nb], zero above the diagonal
    when causal.  The mean runs over the block's queries (fewer in a last
    partial block), the sums over its keys inside the sequence."""
    bk, L = prm.block, prm.seq_len
    t = np.arange(row * bk, min((row + 1) * bk, L))
    n_keys = min((row + 1) * bk, L) if prm.causal else L
    qb = np.asarray(q[b, h, t], dtype=np.float64)
    keys = np.asarray(k[b, h // prm.group, :n_keys], dtype=np.float64)
    s = prm.scale * (qb @ keys.T)  # [rows, n_keys]
    if prm.causal:
        s[np.arange(n_keys)[None, :] > t[:, None]] = -np.inf
    e = np.exp(s - np.max(s, axis=1, keepdims=True))
    p = e / np.sum(e, axis=1, keepdims=True)
    nbk = -(-n_keys // bk)
    pp = np.zeros((t.size, nbk * bk))
    pp[:, :n_keys] = p
    out = np.zeros(prm.num_blocks)
    out[:nbk] = pp.reshape(t.size, nbk, bk).sum(axis=(0, 2)) / t.size
    return out


# ---------------------------------------------------------------------------
# §3.3: Top-tau selection with last-query-block protection (§4.3).
# ---------------------------------------------------------------------------
def top_tau_row(m_row: np.ndarray, row: int, tau: float, protect: bool, causal: bool = True) -> np.ndarray:
    """Selected key blocks (ascending) of query-block row `row`.

    Candidates are J = 0..row (causal) or every key block.  Keep all of them
    if tau >= 1, the row is protected, or the row has no estimate (zero
    total: a last partial block without a sampled query); otherwise sort by
    (mass desc, J asc) and keep the shortest prefix whose cumulative mass
    reaches tau times the row total.
    """
    n = row + 1 if causal else len(m_row)
    if tau >= 1.0 or protect:
        return np.arange(n, dtype=np.int64)
    vals = np.asarray(m_row[:n], dtype=np.float64)
    total = np.sum(vals)
    if not total > 0:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -vals))  # last key is primary: mass desc, then J asc
    csum = np.cumsum(vals[order])
    hit = np.nonzero(csum >= tau * total)[0]
    k_star = int(hit[0]) + 1 if hit.size else n
    return np.sort(order[:k_star])


def select_blocks(m: np.ndarray, prm: Params):
    """Block mask [Bz,H,Nb,Nb] u8, index lists [Bz,H,Nb,Nb] i32 and counts [Bz,H,Nb] i32."""
    nb = prm.num_blocks
    mask = np.zeros((prm.batch, prm.num_heads, nb, nb), dtype=np.uint8)
    idx = np.full((prm.batch, prm.num_heads, nb, nb), -1, dtype=np.int32)
    cnt = np.zeros((prm.batch, prm.num_heads, nb), dtype=np.int32)
    for b in range(prm.batch):
        for h in range(prm.num_heads):
            for i in range(nb):
                sel = top_tau_row(m[b, h, i], i, prm.tau, prm.protect_last and i == nb - 1, prm.causal)
                mask[b, h, i, sel] = 1
                idx[b, h, i, : sel.size] = sel
                cnt[b, h, i] = sel.size
    return mask, idx, cnt


def estimate(q, k, prm: Params, kagg_round: str = "bf16"):
    """Whole estimator: returns (mask, idx, cnt, M)."""
    m = block_scores(q, k, prm, kagg_round)
    mask, idx, cnt = select_blocks(m, prm)
    return mask, idx, cnt, m


# ---------------------------------------------------------------------------
# §4.1: block-sparse causal prefill attention and its dense baseline.
# ---------------------------------------------------------------------------
def _attend(qb: np.ndarray, keys: np.ndarray, vals: np.ndarray, key_pos: np.ndarray,
            q_pos: np.ndarray, sm_scale: float, causal: bool = True) -> np.ndarray:
    """Exact softmax attention of queries qb over the given keys, causally masked."""
    s = sm_scale * (qb @ keys.T)
    if causal:
        s[key_pos[None, :] > q_pos[:, None]] = -np.inf
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    return (e @ vals) / np.sum(e, axis=1, keepdims=True)


def attention_rows(q, k, v, mask, prm: Params, b: int, h: int, row: int) -> np.ndarray:
    """Output rows of query block `row` of head h, restricted to mask[b, h, row].

    Query t attends to keys u <= t (any u when not causal) lying in a
    selected key block and inside the sequence.  Returns [rows, d] float64,
    rows = the block's tokens (fewer for a last partial block).
    """
    bk, L = prm.block, prm.seq_len
    g = h // prm.group
    n_cand = row + 1 if prm.causal else prm.num_blocks
    sel = np.nonzero(np.asarray(mask[b, h, row][:n_cand]))[0]
    if sel.size == 0:
        raise ValueError("empty selection")
    key_pos = (sel[:, None] * bk + np.arange(bk)[None, :]).reshape(-1)
    key_pos = key_pos[key_pos < L]
    q_pos = row * bk + np.arange(bk)
    q_pos = q_pos[q_pos < L]
    qb = np.asarray(q[b, h, q_pos], dtype=np.float64)
    keys = np.asarray(k[b, g, key_pos], dtype=np.float64)
    vals = np.asarray(v[b, g, key_pos], dtype=np.float64)
    return _attend(qb, keys, vals, key_pos, q_pos, prm.scale, prm.causal)


def block_sparse_attention(q, k, v, mask, prm: Params) -> np.ndarray:
    """O[b, h] for every query block, over the selected key blocks only."""
    out = np.zeros((prm.batch, prm.num_heads, prm.seq_len, prm.head_dim))
    bk = prm.block
    for b in range(prm.batch):
        for h in range(prm.num_heads):
            for i in range(prm.num_blocks):
                o = attention_rows(q, k, v, mask, prm, b, h, i)
                out[b, h, i * bk:i * bk + o.shape[0]] = o
    return out


def dense_attention(q, k, v, prm: Params) -> np.ndarray:
    """Dense attention: every causal key block (every key block when not causal) selected."""
    nb = prm.num_blocks
    full = np.ones((nb, nb), dtype=np.uint8)
    if prm.causal:
        full = np.tril(full)
    return block_sparse_attention(q, k, v, np.broadcast_to(full, (prm.batch, prm.num_heads, nb, nb)), prm)
