"""The C ABI library loads on a machine without a GPU, exports every symbol
the header declares, and its host-side checks return the documented status
codes.  Nothing here launches a kernel: every call below fails validation
before any HIP call is made."""
import ctypes
import os
import re

import pytest

import dynamic_block_sparse_sample_amd as rra
from dynamic_block_sparse_sample_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rra.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="librra.so not built")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(rra_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = header_functions()
    assert len(names) == 15, names
    lib = rra.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, n
    assert set(_lib.SIGNATURES) == set(names)


def test_params_struct_matches_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct rra_params \{(.*?)\} rra_params_t;", text, flags=re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [n for n, _ in rra.Params._fields_]
    for (ty, _), (_, cty) in zip(fields, rra.Params._fields_):
        assert cty == (ctypes.c_int32 if ty == "int32_t" else ctypes.c_float)
    assert ctypes.sizeof(rra.Params) == 56


def test_abi_version_and_status_strings():
    assert rra.lib().rra_abi_version() == 3
    for code in range(5):
        assert rra.status_str(code).startswith("RRA_")
    assert rra.status_str(99) == "RRA_ERR_UNKNOWN"


def P(**kw):
    base = dict(batch=1, num_heads=32, num_kv_heads=8, seq_len=8192, head_dim=128, stride=16, block=128,
                tau=0.9, protect_last=True, sm_scale=0.0, causal=True)
    base.update(kw)
    return rra.make_params(**base)


@pytest.mark.parametrize("kw,code", [
    ({}, 0),
    (dict(head_dim=64, block=64, stride=8, seq_len=1024, num_heads=4, num_kv_heads=4), 0),
    (dict(num_heads=28, num_kv_heads=4, seq_len=65536, tau=0.95), 0),
    (dict(stride=4), 0),
    (dict(stride=128), 0),
    (dict(tau=1.0), 0),
    (dict(batch=0), 0),  # empty problem: valid no-op
    (dict(seq_len=0), 0),
    (dict(batch=-1), 1),
    (dict(num_heads=30), 1),  # H % Hkv != 0
    (dict(tau=0.0), 1),
    (dict(tau=1.5), 1),
    (dict(tau=float("nan")), 1),
    (dict(sm_scale=float("inf")), 1),
    (dict(stride=3), 1),  # Bk % S != 0
    (dict(stride=0), 1),
    (dict(num_kv_heads=0), 1),
    (dict(head_dim=96), 2),
    (dict(block=256, stride=16), 2),
    (dict(seq_len=8000), 0),  # ragged: Nb = ceil(L / Bk)
    (dict(seq_len=1), 0),
    (dict(seq_len=128 * 4096 + 1), 2),  # ceil(L / Bk) = 4097 blocks
    (dict(stride=2), 2),  # Bk / S = 64 > 32
    (dict(causal=False), 0),
    (dict(seq_len=128 * 4097), 2),  # more than 4096 blocks
    (dict(rr_mode="layer", rr_layer=31), 0),
    (dict(rr_mode="hybrid", rr_layer=7), 0),
    (dict(rr_mode="none", rr_offset=15), 0),
    (dict(rr_mode=4), 1),
    (dict(rr_mode=-1), 1),
    (dict(rr_layer=-1), 1),
    (dict(rr_mode="none", rr_offset=16), 1),  # offset must lie inside the stride
    (dict(rr_offset=-1), 1),
])
def test_validate_status_codes(kw, code):
    assert rra.validate(P(**kw)) == code


def test_protect_last_must_be_boolean():
    p = P()
    p.protect_last = 2
    assert rra.validate(p) == 1


def test_workspace_size_formula():
    p = P()
    nb, ns = 8192 // 128, 8192 // 16
    kagg = 1 * 8 * ns * 128 * 2
    score = 1 * 32 * nb * nb * 4
    r256 = lambda x: (x + 255) // 256 * 256
    assert rra.workspace_size(p) == r256(kagg) + r256(score)
    assert rra.workspace_size(P(batch=0)) == 0
    # ragged: ceil counts (L = 8000: 63 blocks of 128, 500 strides of 16)
    assert rra.workspace_size(P(seq_len=8000)) == r256(1 * 8 * 500 * 128 * 2) + r256(1 * 32 * 63 * 63 * 4)
    assert rra.workspace_size(P(seq_len=8001)) == r256(1 * 8 * 501 * 128 * 2) + r256(1 * 32 * 63 * 63 * 4)
    with pytest.raises(rra.RRAError):
        rra.workspace_size(P(head_dim=96))


def test_entry_points_reject_null_and_misaligned_pointers_without_launching():
    lib = rra.lib()
    p = P()
    null = None
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first
    odd = ctypes.c_void_p((1 << 20) + 2)
    s = None
    by = ctypes.byref
    assert lib.rra_stride_aggregate(by(p), null, fake, s) == 1
    assert lib.rra_stride_aggregate(by(p), odd, fake, s) == 1
    assert lib.rra_block_scores(by(p), fake, null, fake, s) == 1
    assert lib.rra_top_tau(by(p), fake, fake, null, fake, s) == 1
    assert lib.rra_sparse_attn(by(p), fake, fake, fake, fake, null, fake, null, 0, s) == 1
    assert lib.rra_dense_attn(by(p), fake, fake, fake, odd, null, 0, s) == 1
    assert lib.rra_block_mass(by(p), fake, null, fake, s) == 1
    assert lib.rra_block_mass(by(p), fake, fake, odd, s) == 1
    assert lib.rra_block_mass(by(P(head_dim=96)), fake, fake, fake, s) == 2
    assert lib.rra_xattn_block_scores(by(p), null, fake, fake, s) == 1
    assert lib.rra_xattn_block_scores(by(P(stride=32)), fake, fake, fake, s) == 2  # r = 4: not built
    assert lib.rra_xattn_block_scores(by(P(seq_len=8000)), fake, fake, fake, s) == 2  # ragged
    assert lib.rra_xattn_block_scores(by(P(causal=False)), fake, fake, fake, s) == 2
    assert lib.rra_cast_f32_to_bf16(null, fake, 16, s) == 1
    assert lib.rra_cast_f32_to_bf16(fake, fake, -1, s) == 1
    assert lib.rra_cast_f32_to_bf16(null, null, 0, s) == 0  # nothing to do
    # workspace missing / too small
    assert lib.rra_estimate(by(p), fake, fake, null, 0, fake, fake, fake, null, s) == 3
    need = rra.workspace_size(p)
    assert lib.rra_estimate(by(p), fake, fake, fake, need - 1, fake, fake, fake, null, s) == 3
    # invalid parameters win over everything else
    bad = P(head_dim=96)
    assert lib.rra_estimate(by(bad), fake, fake, fake, 1 << 40, fake, fake, fake, null, s) == 2
    assert lib.rra_dense_attn(None, fake, fake, fake, fake, null, 0, s) == 1
    # the attention calls' optional schedule workspace: too small or misaligned
    wneed = rra.attn_workspace_size(p)
    assert lib.rra_sparse_attn(by(p), fake, fake, fake, fake, fake, fake, fake, wneed - 1, s) == 3
    assert lib.rra_sparse_attn(by(p), fake, fake, fake, fake, fake, fake, odd, wneed, s) == 3
    assert lib.rra_dense_attn(by(p), fake, fake, fake, fake, fake, 0, s) == 3
    assert lib.rra_dense_attn(by(bad), fake, fake, fake, fake, fake, 0, s) == 2


def test_attn_workspace_size():
    """The attention schedule needs one 128-byte counter line per XCD (8), for any valid problem."""
    assert rra.attn_workspace_size(P()) == 1024
    assert rra.attn_workspace_size(P(seq_len=8001, causal=False)) == 1024
    assert rra.attn_workspace_size(P(batch=0)) == 1024
    with pytest.raises(rra.RRAError):
        rra.attn_workspace_size(P(head_dim=96))


def test_empty_problem_is_a_no_op_even_with_null_pointers():
    lib = rra.lib()
    p = P(batch=0)
    by = ctypes.byref
    assert lib.rra_estimate(by(p), None, None, None, 0, None, None, None, None, None) == 0
    assert lib.rra_sparse_attn(by(p), None, None, None, None, None, None, None, 0, None) == 0
    assert lib.rra_dense_attn(by(p), None, None, None, None, None, 0, None) == 0
    assert lib.rra_stride_aggregate(by(p), None, None, None) == 0
    assert lib.rra_block_scores(by(p), None, None, None, None) == 0
    assert lib.rra_top_tau(by(p), None, None, None, None, None) == 0
    assert lib.rra_block_mass(by(p), None, None, None, None) == 0
    assert lib.rra_xattn_block_scores(by(p), None, None, None, None) == 0


def test_header_compiles_as_c_and_host_calls_work(tmp_path):
    """include/rra.h compiles as strict C11 and a C program linked against
    librra.so gets the documented results from the host-only entry points."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    src = os.path.join(ROOT, "tests", "c_abi", "host_calls.c")
    exe = str(tmp_path / "host_calls")
    libdir = os.path.dirname(_lib.LIB_PATH)
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
           src, "-o", exe, f"-L{libdir}", "-lrra", f"-Wl,-rpath,{libdir}"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert run.stdout.strip() == "ok"


def test_binding_workspace_checks_on_host():
    """Workspaces handed to the binding are sized in bytes whatever their dtype,
    and a host tensor is refused before any pointer reaches the library."""
    import torch
    with pytest.raises(ValueError, match="device tensor"):
        _lib._workspace_bytes(torch.empty(1024, dtype=torch.uint8), "workspace")
    with pytest.raises(TypeError):
        _lib._workspace_bytes(bytearray(16), "workspace")
