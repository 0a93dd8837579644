"""Seeded synthetic inputs for RRAttention prefill workloads.

This module only builds Q, K, V (and names the sparsity settings that go with
them).  It holds none of the method's arithmetic, so the CPU oracle and the
HIP path can both be fed from it.

The shapes follow the attention layers of the models the RRAttention page
evaluates (§4.1: Llama-3.1-8B-Instruct, Qwen2-VL-7B-Instruct), at 8K-128K
tokens; the page's datasets (HELMET, Video-MME) are stood in for by planted
structure that puts attention mass where those workloads put it: sink
columns, local diagonals, slash bands, frame-periodic slashes.  Everything is
drawn on the host with a seeded torch.Generator, built in float32 and rounded
to bfloat16 (round to nearest even).

Planting primitives (channel indices count from 0):

* bias channel: for query head h of KV group g, slot hh = h mod G owns
  channel c = d - 1 - hh.  Q[h, :, c] is set to 1 when the head carries the
  pattern, and every other slot's channel of that head is set to 0; K[g, u, c]
  is beta / sm_scale on the planted key tokens u and 0 elsewhere.  The logit of
  (t, u) then gains +beta exactly (up to bf16 rounding) for that head only.
* rotary band: channels [0, 2m) hold m = 32 rotating pairs with frequencies
  w_k = pi * U_k / width and per-head phases phi_{h,k}.  Q[h, t] gets
  a * (cos(w_k t + phi), sin(w_k t + phi)) and K[g, u] gets the same, summed
  over the heads of the group, evaluated at u + delta_h.  The logit of head h
  then holds sm_scale * a^2 * sum_k cos(w_k (t - u - delta_h)): a band of
  width ~ width at offset delta_h, peak sm_scale * a^2 * m.
* periodic codebook (video): one pattern E [256, 64] ~ N(0, 1) on channels
  [0, 64); video token t gets a * E[t mod 256] in Q and K, so logits peak on
  t = u (mod 256).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "headline"]


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    num_heads: int
    num_kv_heads: int
    seq_len: int
    head_dim: int
    stride: int
    block: int
    tau: float
    fp32_inputs: bool = False
    seed: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    # Tiny causal self-attention: 1 x 4 heads (4 KV heads) x 1024 x 64, fp32 draw.
    "tiny_1k": Workload("tiny_1k", 1, 4, 4, 1024, 64, 8, 64, 0.9, fp32_inputs=True),
    # Llama-3-8B attention layer (32 q heads, 8 KV heads, d=128) at 8K.
    "llama_8k": Workload("llama_8k", 1, 32, 8, 8192, 128, 16, 128, 0.9),
    # Same layer at 32K with mixed per-head structure; S and tau are swept.
    "llama_32k": Workload("llama_32k", 1, 32, 8, 32768, 128, 16, 128, 0.9),
    # Same layer at 128K: the headline sparse-vs-dense comparison.
    "llama_128k": Workload("llama_128k", 1, 32, 8, 131072, 128, 16, 128, 0.9),
    # Qwen2-VL-7B attention layer (28 q heads, 4 KV heads) on 64K video tokens.
    "video_64k": Workload("video_64k", 1, 28, 4, 65536, 128, 16, 128, 0.95),
}

# Headline-workload constants: sink logit bias and slash-band amplitude.
# Chosen so that the mask density at tau = 0.9 is about one half, the share of
# blocks the RRAttention page reports computing (§4.2).
HEADLINE_SINK_BETA = 4.0
HEADLINE_BAND_PEAK = 5.0


def headline() -> Workload:
    return WORKLOADS["llama_128k"]


# ---------------------------------------------------------------------------
def _slot_channel(d: int, group: int, h: int) -> int:
    return d - 1 - (h % group)


def _plant_bias(q, k, group, sm_scale, heads_betas_cols):
    """heads_betas_cols: list of (head, beta, key token indices)."""
    d = q.shape[-1]
    H = q.shape[1]
    # every head sees only its own slot channel
    for h in range(H):
        for hh in range(group):
            q[:, h, :, d - 1 - hh] = 0.0
    k[:, :, :, d - group:] = 0.0
    for h, beta, cols in heads_betas_cols:
        c = _slot_channel(d, group, h)
        q[:, h, :, c] = 1.0
        k[:, h // group, cols, c] = beta / sm_scale


def _plant_band(q, k, group, sm_scale, peak, width, deltas, gen, heads=None, m=32):
    """Rotary band on channels [0, 2m) for the listed heads (default: all)."""
    B, H, L, d = q.shape
    heads = list(range(H)) if heads is None else list(heads)
    a = math.sqrt(peak / (sm_scale * m))
    U = torch.rand(m, generator=gen, dtype=torch.float64)
    omega = math.pi * U / width  # [m]
    phi = torch.rand(H, m, generator=gen, dtype=torch.float64) * (2 * math.pi)
    t = torch.arange(L, dtype=torch.float64)
    for h in heads:
        ang_q = t[:, None] * omega[None, :] + phi[h][None, :]  # [L, m]
        q[:, h, :, 0:2 * m:2] += (a * torch.cos(ang_q)).float()
        q[:, h, :, 1:2 * m:2] += (a * torch.sin(ang_q)).float()
        ang_k = (t[:, None] + float(deltas[h])) * omega[None, :] + phi[h][None, :]
        g = h // group
        k[:, g, :, 0:2 * m:2] += (a * torch.cos(ang_k)).float()
        k[:, g, :, 1:2 * m:2] += (a * torch.sin(ang_k)).float()


def make_inputs(w: Workload, device="cpu", structure: bool = True):
    """Seeded Q [Bz,H,L,d], K, V [Bz,Hkv,L,d] as bfloat16 (float32 for fp32 draws).

    Drawn in the order Q, K, V, then structure randomness, from one
    torch.Generator seeded with w.seed.  For fp32 workloads the float32
    tensors are returned (the library rounds them to bf16 at its boundary).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed)
    B, H, Hkv, L, d = w.batch, w.num_heads, w.num_kv_heads, w.seq_len, w.head_dim
    G = H // Hkv
    sc = w.sm_scale
    q = torch.randn(B, H, L, d, generator=gen, dtype=torch.float32)
    k = torch.randn(B, Hkv, L, d, generator=gen, dtype=torch.float32)
    v = torch.randn(B, Hkv, L, d, generator=gen, dtype=torch.float32)
    name = w.name
    if name in ("llama_8k", "llama_32k", "video_64k"):
        q /= math.sqrt(d)
        k /= math.sqrt(d)
        v /= math.sqrt(d)
    if structure:
        if name == "tiny_1k":
            # local diagonal: each key carries 3x its own token's query (G = 1),
            # then a vertical column at token 0 through the bias channel.
            k += 3.0 * q
            _plant_bias(q, k, G, sc, [(h, 4.0 * w.stride, [0]) for h in range(H)])
        elif name == "llama_8k":
            _plant_band(q, k, G, sc, 6.0, 128.0, [0] * H, gen)
            _plant_bias(q, k, G, sc, [(h, 8.0, [0, 1, 2, 3]) for h in range(H)])
        elif name == "llama_32k":
            even = [h for h in range(H) if h % 2 == 0]
            _plant_band(q, k, G, sc, 6.0, 128.0, [0] * H, gen, heads=even)
            plants = []
            for h in range(H):
                if h % 2 == 1:
                    cols = torch.randint(0, L, (16,), generator=gen).tolist()
                    plants.append((h, 4.0, cols))
            _plant_bias(q, k, G, sc, plants)
        elif name == "llama_128k":
            deltas = torch.randint(0, 16384, (H,), generator=gen).tolist()
            _plant_band(q, k, G, sc, HEADLINE_BAND_PEAK, 128.0, deltas, gen)
            _plant_bias(q, k, G, sc, [(h, HEADLINE_SINK_BETA, [0, 1, 2, 3]) for h in range(H)])
        elif name == "video_64k":
            frames, ftok, m2 = 254, 256, 64
            nvid = frames * ftok
            E = torch.randn(ftok, m2, generator=gen, dtype=torch.float32)
            a = math.sqrt(6.0 / (sc * m2))
            pat = E.repeat(frames, 1)  # [nvid, 64]
            q[:, :, :nvid, :m2] += a * pat
            k[:, :, :nvid, :m2] += a * pat
        else:
            raise ValueError(f"no structure recipe for {name}")
    if w.fp32_inputs:
        return q.to(device), k.to(device), v.to(device)
    return (q.to(torch.bfloat16).to(device), k.to(torch.bfloat16).to(device),
            v.to(torch.bfloat16).to(device))


def make_random(batch, num_heads, num_kv_heads, seq_len, head_dim, seed=0, scale=1.0, diag=0.0):
    """Seeded N(0, scale^2) Q, K, V as bfloat16 on the host.

    diag > 0 adds diag * Q[head 0 of the group] to K, a token-aligned local
    diagonal that gives the selection some structure.
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = torch.randn(batch, num_heads, seq_len, head_dim, generator=gen) * scale
    k = torch.randn(batch, num_kv_heads, seq_len, head_dim, generator=gen) * scale
    v = torch.randn(batch, num_kv_heads, seq_len, head_dim, generator=gen)
    if diag:
        G = num_heads // num_kv_heads
        k += diag * q[:, ::G]
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
