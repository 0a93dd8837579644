"""ctypes binding of librra.so (the C ABI declared in include/rra.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  There is
no fallback: if librra.so is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librra.so")

RRA_OK = 0
RRA_ERR_INVALID_ARG = 1
RRA_ERR_UNSUPPORTED = 2
RRA_ERR_WORKSPACE = 3
RRA_ERR_HIP = 4

# Every function the header declares, with its ctypes signature.
_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class Params(ctypes.Structure):
    """Mirror of rra_params_t."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("stride", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("protect_last", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("rr_mode", ctypes.c_int32),
        ("rr_layer", ctypes.c_int32),
        ("rr_offset", ctypes.c_int32),
    ]

    def __repr__(self):
        return "Params(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"

    @property
    def num_blocks(self) -> int:
        return -(-self.seq_len // self.block) if self.block > 0 else 0  # ceil: a last partial block counts

    @property
    def num_strides(self) -> int:
        return -(-self.seq_len // self.stride) if self.stride > 0 else 0


SIGNATURES = {
    "rra_abi_version": (ctypes.c_int, []),
    "rra_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "rra_validate": (ctypes.c_int, [ctypes.POINTER(Params)]),
    "rra_estimate_workspace_size": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_size_t)]),
    "rra_cast_f32_to_bf16": (ctypes.c_int, [_P, _P, ctypes.c_int64, _P]),
    "rra_stride_aggregate": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P]),
    "rra_block_scores": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P]),
    "rra_top_tau": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P, _P]),
    "rra_estimate": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, ctypes.c_size_t, _P, _P, _P, _P, _P]),
    "rra_estimate_noalloc": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P]),
    "rra_block_mass": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P]),
    "rra_xattn_block_scores": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P]),
    "rra_sparse_attn": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "rra_dense_attn": (ctypes.c_int, [ctypes.POINTER(Params), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "rra_attn_workspace_size": (ctypes.c_int, [ctypes.POINTER(Params), ctypes.POINTER(ctypes.c_size_t)]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load librra.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m dynamic_block_sparse_sample_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_str(code: int) -> str:
    return lib().rra_status_str(code).decode()


class RRAError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {status_str(code)}")
        self.code = code


def _check(fn: str, code: int) -> None:
    if code != RRA_OK:
        raise RRAError(fn, code)


# Round-robin strategies (rra_rr_mode_t): offset of the sampled query inside a stride.
RR_MODES = {"head": 0, "layer": 1, "hybrid": 2, "none": 3}


def make_params(batch, num_heads, num_kv_heads, seq_len, head_dim, stride, block, tau,
                protect_last=True, sm_scale=0.0, causal=True, rr_mode="head", rr_layer=0,
                rr_offset=0) -> Params:
    return Params(int(batch), int(num_heads), int(num_kv_heads), int(seq_len), int(head_dim), int(stride),
                  int(block), float(tau), int(bool(causal)), int(bool(protect_last)), float(sm_scale),
                  RR_MODES[rr_mode] if isinstance(rr_mode, str) else int(rr_mode), int(rr_layer),
                  int(rr_offset))


def validate(p: Params) -> int:
    return lib().rra_validate(ctypes.byref(p))


def workspace_size(p: Params) -> int:
    n = ctypes.c_size_t(0)
    _check("rra_estimate_workspace_size", lib().rra_estimate_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _on(stream):
    """Context in which the binding allocates what a call needs (workspaces,
    default outputs): the launch stream, so that torch's caching allocator
    never hands those bytes to other work before the call's kernels finish."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace_bytes(t: torch.Tensor, name: str) -> int:
    """Size in bytes of a caller-supplied workspace (any dtype): a contiguous device tensor."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.numel() * t.element_size()


def _shapes(p: Params):
    q = (p.batch, p.num_heads, p.seq_len, p.head_dim)
    kv = (p.batch, p.num_kv_heads, p.seq_len, p.head_dim)
    return q, kv, p.num_blocks, p.num_strides


def cast_f32_to_bf16(src: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _need(src, "src", torch.float32, src.shape)
    if out is None:
        with _on(stream):
            out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.device)
    _need(out, "out", torch.bfloat16, src.shape)
    _check("rra_cast_f32_to_bf16", lib().rra_cast_f32_to_bf16(_ptr(src), _ptr(out), src.numel(), _stream(stream)))
    return out


def stride_aggregate(p: Params, k: torch.Tensor, kagg: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _, kv, _, ns = _shapes(p)
    _need(k, "k", torch.bfloat16, kv)
    if kagg is None:
        with _on(stream):
            kagg = torch.empty((p.batch, p.num_kv_heads, ns, p.head_dim), dtype=torch.bfloat16, device=k.device)
    _need(kagg, "kagg", torch.bfloat16, (p.batch, p.num_kv_heads, ns, p.head_dim))
    _check("rra_stride_aggregate", lib().rra_stride_aggregate(ctypes.byref(p), _ptr(k), _ptr(kagg), _stream(stream)))
    return kagg


def block_scores(p: Params, q: torch.Tensor, kagg: torch.Tensor, score: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    qs, _, nb, ns = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(kagg, "kagg", torch.bfloat16, (p.batch, p.num_kv_heads, ns, p.head_dim))
    if score is None:
        with _on(stream):
            score = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=q.device)
    _need(score, "score", torch.float32, (p.batch, p.num_heads, nb, nb))
    _check("rra_block_scores",
           lib().rra_block_scores(ctypes.byref(p), _ptr(q), _ptr(kagg), _ptr(score), _stream(stream)))
    return score


def block_mass(p: Params, q: torch.Tensor, k: torch.Tensor, mass: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
    """Exact block masses of full causal attention, float32 [Bz, H, Nb, Nb]."""
    qs, ks, nb, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, ks)
    if mass is None:
        with _on(stream):
            mass = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=q.device)
    _need(mass, "mass", torch.float32, (p.batch, p.num_heads, nb, nb))
    _check("rra_block_mass", lib().rra_block_mass(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(mass), _stream(stream)))
    return mass


def xattn_block_scores(p: Params, q: torch.Tensor, k: torch.Tensor, score: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """XAttention's antidiagonal block scores (the comparison estimator), float32 [Bz, H, Nb, Nb]."""
    qs, ks, nb, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, ks)
    if score is None:
        with _on(stream):
            score = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=q.device)
    _need(score, "score", torch.float32, (p.batch, p.num_heads, nb, nb))
    _check("rra_xattn_block_scores",
           lib().rra_xattn_block_scores(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(score), _stream(stream)))
    return score


def _selection_buffers(p: Params, device, mask=None, idx=None, cnt=None, stream=None):
    _, _, nb, _ = _shapes(p)
    with _on(stream):
        if mask is None:
            mask = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.uint8, device=device)
        if idx is None:
            idx = torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.int32, device=device)
        if cnt is None:
            cnt = torch.empty((p.batch, p.num_heads, nb), dtype=torch.int32, device=device)
    _need(mask, "mask", torch.uint8, (p.batch, p.num_heads, nb, nb))
    _need(idx, "idx", torch.int32, (p.batch, p.num_heads, nb, nb))
    _need(cnt, "cnt", torch.int32, (p.batch, p.num_heads, nb))
    return mask, idx, cnt


def top_tau(p: Params, score: torch.Tensor, mask=None, idx=None, cnt=None, stream=None):
    _, _, nb, _ = _shapes(p)
    _need(score, "score", torch.float32, (p.batch, p.num_heads, nb, nb))
    mask, idx, cnt = _selection_buffers(p, score.device, mask, idx, cnt, stream)
    _check("rra_top_tau", lib().rra_top_tau(ctypes.byref(p), _ptr(score), _ptr(mask), _ptr(idx), _ptr(cnt),
                                            _stream(stream)))
    return mask, idx, cnt


@dataclass
class Selection:
    mask: torch.Tensor
    idx: torch.Tensor
    cnt: torch.Tensor
    score: torch.Tensor | None


def alloc_workspace(p: Params, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_size(p), 1), dtype=torch.uint8, device=device)


def estimate(p: Params, q: torch.Tensor, k: torch.Tensor, workspace: torch.Tensor | None = None,
             return_score: bool = False, out: Selection | None = None, stream=None) -> Selection:
    qs, kv, nb, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, kv)
    if workspace is None:
        with _on(stream):
            workspace = alloc_workspace(p, q.device)
    if out is None:
        mask, idx, cnt = _selection_buffers(p, q.device, stream=stream)
        with _on(stream):
            score = (torch.empty((p.batch, p.num_heads, nb, nb), dtype=torch.float32, device=q.device)
                     if return_score else None)
        out = Selection(mask, idx, cnt, score)
    _selection_buffers(p, q.device, out.mask, out.idx, out.cnt)
    if out.score is not None:
        _need(out.score, "score", torch.float32, (p.batch, p.num_heads, nb, nb))
    ws_bytes = _workspace_bytes(workspace, "workspace")
    _check("rra_estimate",
           lib().rra_estimate(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(workspace), ws_bytes,
                              _ptr(out.mask), _ptr(out.idx), _ptr(out.cnt), _ptr(out.score), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # RRA_NOALLOC_SCRATCH_BYTES


def estimate_noalloc(p: Params, q: torch.Tensor, k: torch.Tensor, out: Selection, stream=None) -> Selection:
    """rra_estimate_noalloc: the estimator with its intermediates in the
    library's own device array (no workspace).  `out` supplies every output
    buffer (the binding allocates nothing here either)."""
    qs, kv, nb, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, kv)
    _selection_buffers(p, q.device, out.mask, out.idx, out.cnt)
    if out.score is not None:
        _need(out.score, "score", torch.float32, (p.batch, p.num_heads, nb, nb))
    _check("rra_estimate_noalloc",
           lib().rra_estimate_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(out.mask), _ptr(out.idx),
                                      _ptr(out.cnt), _ptr(out.score), _stream(stream)))
    return out


def attn_workspace_size(p: Params) -> int:
    n = ctypes.c_size_t(0)
    _check("rra_attn_workspace_size", lib().rra_attn_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def _attn_workspace(p: Params, device, workspace, schedule: str, stream=None):
    """(pointer, bytes) of the schedule workspace: a fresh one per call unless given
    (calls that may overlap need distinct ones); (None, 0) for schedule="static"."""
    if schedule == "static":
        return None, 0
    if schedule != "dynamic":
        raise ValueError(f"schedule must be 'dynamic' or 'static', not {schedule!r}")
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(attn_workspace_size(p), dtype=torch.uint8, device=device)
    return _ptr(workspace), _workspace_bytes(workspace, "workspace")


def sparse_attn(p: Params, q, k, v, idx, cnt, out=None, workspace=None, schedule="dynamic",
                stream=None) -> torch.Tensor:
    """Block-sparse attention on the selected key blocks.  schedule="dynamic" (a
    per-call workspace unless one is given) balances the rows over the XCDs;
    "static" runs one workgroup per row.  Both give bitwise the same output."""
    qs, kv, nb, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, kv)
    _need(v, "v", torch.bfloat16, kv)
    _need(idx, "idx", torch.int32, (p.batch, p.num_heads, nb, nb))
    _need(cnt, "cnt", torch.int32, (p.batch, p.num_heads, nb))
    if out is None:
        with _on(stream):
            out = torch.empty(qs, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, qs)
    ws, ws_bytes = _attn_workspace(p, q.device, workspace, schedule, stream)
    _check("rra_sparse_attn", lib().rra_sparse_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                                    _ptr(cnt), _ptr(out), ws, ws_bytes, _stream(stream)))
    return out


def dense_attn(p: Params, q, k, v, out=None, workspace=None, schedule="dynamic", stream=None) -> torch.Tensor:
    qs, kv, _, _ = _shapes(p)
    _need(q, "q", torch.bfloat16, qs)
    _need(k, "k", torch.bfloat16, kv)
    _need(v, "v", torch.bfloat16, kv)
    if out is None:
        with _on(stream):
            out = torch.empty(qs, dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, qs)
    ws, ws_bytes = _attn_workspace(p, q.device, workspace, schedule, stream)
    _check("rra_dense_attn", lib().rra_dense_attn(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), ws,
                                                  ws_bytes, _stream(stream)))
    return out
