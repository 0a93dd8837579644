"""RRAttention block-sparse causal prefill attention for AMD MI355X (gfx950).

The compute runs in librra.so (hand-written HIP kernels behind the C ABI in
include/rra.h); this package is its Python binding plus seeded workload
generators.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    Params,
    RRAError,
    Selection,
    alloc_workspace,
    attn_workspace_size,
    block_mass,
    block_scores,
    cast_f32_to_bf16,
    dense_attn,
    estimate,
    estimate_noalloc,
    lib,
    make_params,
    sparse_attn,
    status_str,
    stride_aggregate,
    top_tau,
    validate,
    workspace_size,
    xattn_block_scores,
)

__all__ = [
    "LIB_PATH", "Params", "RRAError", "Selection", "alloc_workspace", "attn_workspace_size", "block_mass",
    "block_scores",
    "cast_f32_to_bf16",
    "dense_attn", "estimate", "estimate_noalloc", "lib", "make_params", "sparse_attn", "status_str", "stride_aggregate",
    "top_tau", "validate", "workspace_size", "xattn_block_scores",
]
