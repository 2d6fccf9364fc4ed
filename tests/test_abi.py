"""C-ABI checks that need no GPU: the library loads, exports every function
include/normrope.h declares, and its host-side logic (argument checks, status
strings, workspace sizing, tuning keys) behaves as documented.  No call here
reaches a kernel launch: each either is host-only or fails validation first.
"""
import ctypes
import os
import re
import subprocess

import pytest

import rmsnorm_layernorm_fwd_amd as nr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "normrope.h")

NR_OK, NR_ERR_NULLPTR, NR_ERR_SHAPE, NR_ERR_DTYPE, NR_ERR_UNSUPPORTED_N = 0, 1, 2, 3, 4
NR_ERR_WORKSPACE, NR_ERR_HIP, NR_ERR_ALIAS, NR_ERR_TUNE = 5, 6, 7, 8
F32, BF16, F16 = 0, 1, 2
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return nr._lib()


def test_header_functions_exported(lib):
    names = declared_functions()
    expected = {"rmsnorm_fwd", "rmsnorm_bwd", "layernorm_fwd", "layernorm_bwd",
                "rmsnorm_rope_fwd", "rmsnorm_rope_bwd", "layernorm_gelu_fwd", "layernorm_gelu_bwd",
                "rope_interleaved_apply", "rope_table_1d", "rope_table_3d",
                "nr_bwd_workspace_bytes", "nr_status_str", "nr_last_hip_error", "nr_tune",
                "nr_norm_n_max", "nr_stream_copy", "rmsnorm_linear_fwd",
                "rmsnorm_linear_fold_weight", "nr_rmsnorm_linear_workspace_bytes"}
    assert expected <= set(names), names
    out = subprocess.run(["nm", "-D", "--defined-only", nr.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for n in names:
        assert n in exported, f"{n} declared in normrope.h but not exported"
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for code in range(9):
        s = nr.nr_status_str(code)
        assert s and s != "unknown status"
    assert nr.nr_status_str(99) == "unknown status"
    assert nr.nr_status_str(0) == "ok"


def test_norm_n_max():
    import torch
    assert nr.nr_norm_n_max(torch.bfloat16) == 65536
    assert nr.nr_norm_n_max(torch.float32) == 32768
    assert nr.nr_norm_n_max(torch.float16) == 65536


def test_workspace_bytes():
    # one fp32 partial row per backward workgroup; workgroups take >= 8 rows,
    # at most 256 (RMSNorm) or 512 (LayerNorm) of them, none empty
    assert nr.nr_bwd_workspace_bytes(3840, 5120, 0) == 256 * 5120 * 4
    assert nr.nr_bwd_workspace_bytes(3840, 5120, 1) == 2 * 480 * 5120 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 5120, 0) == 256 * 5120 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 5120, 1) == 2 * 512 * 5120 * 4
    assert nr.nr_bwd_workspace_bytes(15360, 5120, 1) == 2 * 512 * 5120 * 4
    assert nr.nr_bwd_workspace_bytes(1, 7, 0) == 7 * 4
    assert nr.nr_bwd_workspace_bytes(0, 7, 0) == 0
    # 17 rows: 3 workgroups of at most 6 rows
    assert nr.nr_bwd_workspace_bytes(17, 8, 0) == 3 * 8 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 5120, 2) == 512 * 5120 * 4  # fused RMSNorm + RoPE
    assert nr.nr_bwd_workspace_bytes(64, 8, 3) == 0
    # rows of more than 16384 elements: ceil(rows / 16) (at most 128) partial
    # rows, then two fp32 terms per row
    assert nr.nr_bwd_workspace_bytes(100, 20000, 1) == 7 * 20000 * 4 * 2 + 100 * 8
    assert nr.nr_bwd_workspace_bytes(100, 20000, 0) == 7 * 20000 * 4 + 100 * 8
    assert nr.nr_bwd_workspace_bytes(4096, 32768, 2) == 128 * 32768 * 4 + 4096 * 8


def test_linear_workspace_bytes():
    # the 256 x 256 path (N % 256 == 0): the row statistics (M fp32, rounded
    # up to 256 bytes), then the folded weight (N K bf16) when there is a
    # norm weight; nothing on the 128 x 128 path
    rows = lambda m: (m * 4 + 255) // 256 * 256
    assert nr.nr_rmsnorm_linear_workspace_bytes(65536, 5120, 5120, True) == rows(65536) + 5120 * 5120 * 2
    assert nr.nr_rmsnorm_linear_workspace_bytes(65536, 5120, 5120, False) == rows(65536)
    assert nr.nr_rmsnorm_linear_workspace_bytes(65537, 5120, 64, False) == rows(65537)
    assert nr.nr_rmsnorm_linear_workspace_bytes(3840, 5120, 5120, True) == rows(3840) + 5120 * 5120 * 2
    assert nr.nr_rmsnorm_linear_workspace_bytes(1, 256, 64, True) == 256 + 256 * 64 * 2
    assert nr.nr_rmsnorm_linear_workspace_bytes(65536, 5120 + 128, 5120, True) == 0
    assert nr.nr_rmsnorm_linear_workspace_bytes(0, 5120, 5120, True) == 0


def test_tune_keys(lib):
    assert lib.nr_tune(b"bwd_d", 0) == NR_OK
    assert lib.nr_tune(b"no_such_key", 1) == NR_ERR_TUNE
    assert lib.nr_tune(b"fwd_w", -1) == NR_ERR_TUNE
    assert lib.nr_tune(None, 1) == NR_ERR_TUNE
    # a forced workgroup count changes the workspace size, 0 restores it
    assert lib.nr_tune(b"bwd_p", 120) == NR_OK
    try:
        assert nr.nr_bwd_workspace_bytes(3840, 5120, 0) == 120 * 5120 * 4
    finally:
        assert lib.nr_tune(b"bwd_p", 0) == NR_OK
    assert nr.nr_bwd_workspace_bytes(3840, 5120, 0) == 256 * 5120 * 4


def test_rejected_calls_return_status(lib):
    L = lib
    # dtype
    assert L.rmsnorm_fwd(7, FAKE, None, FAKE, None, 4, 8, 1e-6, 0, None) == NR_ERR_DTYPE
    assert L.rope_interleaved_apply(3, FAKE, FAKE, FAKE, 1, 1, 1, 8, 8, 8, 8, 0, None) == NR_ERR_DTYPE
    assert L.layernorm_gelu_fwd(-1, FAKE, None, None, FAKE, None, None, 4, 8, 1e-5, None) == NR_ERR_DTYPE
    # null required pointers
    assert L.rmsnorm_fwd(BF16, None, None, FAKE, None, 4, 8, 1e-6, 0, None) == NR_ERR_NULLPTR
    assert L.rmsnorm_fwd(BF16, FAKE, None, None, None, 4, 8, 1e-6, 0, None) == NR_ERR_NULLPTR
    assert L.rmsnorm_bwd(BF16, FAKE, FAKE, None, None, FAKE, None, 4, 8, 0, None, 0, None) == NR_ERR_NULLPTR
    assert L.layernorm_bwd(F32, FAKE, FAKE, None, None, FAKE, FAKE, None, None, 4, 8, None, 0, None) == NR_ERR_NULLPTR
    assert L.rope_interleaved_apply(F32, FAKE, None, FAKE, 1, 1, 1, 8, 8, 8, 8, 0, None) == NR_ERR_NULLPTR
    assert L.rope_table_1d(None, FAKE, 4, 8, 0, 1e4, None) == NR_ERR_NULLPTR
    # shapes
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAKE, None, 4, 0, 1e-6, 0, None) == NR_ERR_SHAPE
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAKE, None, -1, 8, 1e-6, 0, None) == NR_ERR_SHAPE
    assert L.layernorm_fwd(F32, FAKE, None, None, FAKE, None, None, 4, -3, 1e-5, None) == NR_ERR_SHAPE
    assert L.rope_interleaved_apply(F32, FAKE, FAKE, FAKE, 1, 4, 2, 7, 14, 7, 7, 0, None) == NR_ERR_SHAPE
    assert L.rope_interleaved_apply(F32, FAKE, FAKE, FAKE, 1, 4, 2, 8, -1, 16, 8, 0, None) == NR_ERR_SHAPE
    assert L.rope_table_1d(FAKE, FAKE, 4, 7, 0, 1e4, None) == NR_ERR_SHAPE
    assert L.rope_table_1d(FAKE, FAKE, 4, 8, 0, -1.0, None) == NR_ERR_SHAPE
    assert L.rope_table_3d(FAKE, FAKE, 2, 3, 4, 0, 2, 2, 1e4, None) == NR_ERR_SHAPE
    assert L.rmsnorm_fwd(F16, FAKE, None, None, None, 4, 8, 1e-6, 0, None) == NR_ERR_NULLPTR
    # row length beyond the on-chip limit
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAKE, None, 4, 65537, 1e-6, 0, None) == NR_ERR_UNSUPPORTED_N
    assert L.rmsnorm_fwd(F32, FAKE, None, FAKE, None, 4, 32769, 1e-6, 0, None) == NR_ERR_UNSUPPORTED_N
    assert L.layernorm_bwd(BF16, FAKE, FAKE, None, FAKE, FAKE, FAKE, None, None, 4, 70000, None, 0, None) == NR_ERR_UNSUPPORTED_N
    # partial overlap of an output with an input
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAKE + 2, None, 4, 8, 1e-6, 0, None) == NR_ERR_ALIAS
    assert L.rmsnorm_bwd(BF16, FAKE, 0x90000, None, FAKE, FAKE + 16, None, 4, 8, 0, None, 0, None) == NR_ERR_ALIAS
    assert L.rope_interleaved_apply(BF16, FAKE, FAKE, FAKE, 1, 4, 2, 8, 64, 16, 4, 0, None) == NR_ERR_ALIAS
    # workspace missing, short or misaligned when a column gradient is wanted
    need = nr.nr_bwd_workspace_bytes(64, 256, 0)
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, FAKE, 0xA0000, FAKE, 64, 256, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, FAKE, 0xA0000, FAKE, 64, 256, 0, 0xB0000, need - 4, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, FAKE, 0xA0000, FAKE, 64, 256, 0, 0xB0004, need, None) == NR_ERR_WORKSPACE
    need_ln = nr.nr_bwd_workspace_bytes(64, 256, 1)
    assert L.layernorm_bwd(F32, FAKE, 0x90000, None, FAKE, FAKE, 0xA0000, None, FAKE, 64, 256, 0xB0000, need_ln - 1, None) == NR_ERR_WORKSPACE
    # grids beyond the hardware's 2^31 - 1 workgroups are refused, not truncated
    FAR = 1 << 40
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAR, None, 1 << 33, 1, 1e-6, 0, None) == NR_ERR_SHAPE
    assert L.rope_interleaved_apply(BF16, FAKE, FAR, FAR + (1 << 36), 1, 1 << 33, 1, 2, 2, 2, 2, 0,
                                    None) == NR_ERR_SHAPE
    # RMSNorm -> linear: bf16 only, K % 64, N % 128, pointers, alignment, overlap
    XA, WA, OA = 1 << 24, 1 << 28, 1 << 32
    lin = L.rmsnorm_linear_fwd
    assert lin(F32, XA, None, WA, OA, None, 4, 128, 64, 1e-6, 0, None, 0, None) == NR_ERR_DTYPE
    assert lin(BF16, XA, None, WA, OA, None, 4, 100, 64, 1e-6, 0, None, 0, None) == NR_ERR_SHAPE
    assert lin(BF16, XA, None, WA, OA, None, 4, 128, 72, 1e-6, 0, None, 0, None) == NR_ERR_SHAPE
    assert lin(BF16, XA, None, WA, OA, None, 4, 128, 65600, 1e-6, 0, None, 0, None) == NR_ERR_UNSUPPORTED_N
    assert lin(BF16, None, None, WA, OA, None, 4, 128, 64, 1e-6, 0, None, 0, None) == NR_ERR_NULLPTR
    assert lin(BF16, XA + 2, None, WA, OA, None, 4, 128, 64, 1e-6, 0, None, 0, None) == NR_ERR_SHAPE
    assert lin(BF16, XA, None, WA, XA + 64, None, 4, 128, 64, 1e-6, 0, None, 0, None) == NR_ERR_ALIAS
    assert lin(BF16, None, None, None, None, None, 0, 128, 64, 1e-6, 0, None, 0, None) == NR_OK
    # the 256 x 256 path with a norm weight needs the folded-weight workspace
    # (N K bf16), aligned and apart from the operands
    BX, BW, BO, BN_, BS, BR = 1 << 34, 1 << 36, 1 << 38, 1 << 40, 1 << 41, 1 << 42
    big = (65536, 5120, 64, 1e-6, 0)
    need = 65536 * 4 + 5120 * 64 * 2
    assert lin(BF16, BX, BN_, BW, BO, BR, *big, None, 0, None) == NR_ERR_WORKSPACE
    assert lin(BF16, BX, BN_, BW, BO, BR, *big, BS, need - 16, None) == NR_ERR_WORKSPACE
    assert lin(BF16, BX, BN_, BW, BO, BR, *big, BS + 8, need, None) == NR_ERR_WORKSPACE
    assert lin(BF16, BX, BN_, BW, BO, BR, *big, BW + 1024, need, None) == NR_ERR_ALIAS
    assert lin(BF16, BX, BN_, BW, BO, BR, *big, BR - 1024, need, None) == NR_ERR_ALIAS
    # without a norm weight the workspace holds the row statistics only, and
    # is not needed when inv_rms takes them
    assert lin(BF16, BX, None, BW, BO, None, *big, None, 0, None) == NR_ERR_WORKSPACE
    assert lin(BF16, BX, None, BW, BO, None, *big, BS, 65536 * 4 - 4, None) == NR_ERR_WORKSPACE
    # forcing the 256 x 256 tile where N is not a multiple of 256
    assert L.nr_tune(b"gemm_tile", 2) == NR_OK
    try:
        assert lin(BF16, XA, None, WA, OA, None, 4, 384, 64, 1e-6, 0, None, 0, None) == NR_ERR_SHAPE
    finally:
        L.nr_tune(b"gemm_tile", 0)
    # the standalone fold: bf16, K % 8, pointers, alignment, partial overlap
    fold = L.rmsnorm_linear_fold_weight
    assert fold(F32, XA, WA, OA, 16, 64, 0, None) == NR_ERR_DTYPE
    assert fold(BF16, XA, WA, OA, 16, 60, 0, None) == NR_ERR_SHAPE
    assert fold(BF16, None, WA, OA, 16, 64, 0, None) == NR_ERR_NULLPTR
    assert fold(BF16, XA, WA + 2, OA, 16, 64, 0, None) == NR_ERR_SHAPE
    assert fold(BF16, XA, WA, WA + 128, 16, 64, 0, None) == NR_ERR_ALIAS
    assert fold(BF16, XA, WA, XA, 16, 64, 0, None) == NR_ERR_ALIAS
    assert fold(BF16, None, None, None, 0, 64, 0, None) == NR_OK
    # the copy probe: null, size / alignment, overlap; zero bytes is a no-op
    assert L.nr_stream_copy(None, FAKE, 64, None) == NR_ERR_NULLPTR
    assert L.nr_stream_copy(FAKE, 0x90000, 60, None) == NR_ERR_SHAPE
    assert L.nr_stream_copy(FAKE + 8, 0x90000, 64, None) == NR_ERR_SHAPE
    assert L.nr_stream_copy(FAKE, FAKE + 32, 64, None) == NR_ERR_ALIAS
    assert L.nr_stream_copy(FAKE, FAKE, 64, None) == NR_ERR_ALIAS
    assert L.nr_stream_copy(None, None, 0, None) == NR_OK
    # long rows need the workspace even without a column gradient
    X2, DX2, WS2 = 1 << 24, 1 << 25, 1 << 26
    assert L.rmsnorm_bwd(BF16, FAKE, X2, None, FAKE, DX2, None, 4, 20000, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.layernorm_bwd(F32, FAKE, X2, None, FAKE, FAKE, DX2, None, None, 4, 20000, WS2, 31, None) == NR_ERR_WORKSPACE
    # a forced launch shape that cannot cover the row
    assert L.nr_tune(b"fwd_k", 1) == NR_OK
    try:
        assert L.rmsnorm_fwd(BF16, FAKE, None, FAKE, None, 4, 5120, 1e-6, 0, None) == NR_ERR_SHAPE
    finally:
        L.nr_tune(b"fwd_k", 0)


def test_empty_forward_is_a_noop(lib):
    # rows == 0 / tokens == 0 return before touching the device
    assert lib.rmsnorm_fwd(BF16, None, None, None, None, 0, 8, 1e-6, 0, None) == NR_OK
    assert lib.layernorm_fwd(F32, None, None, None, None, None, None, 0, 8, 1e-5, None) == NR_OK
    assert lib.rope_interleaved_apply(BF16, None, None, None, 1, 0, 4, 8, 0, 0, 0, 0, None) == NR_OK
    assert lib.rope_table_1d(None, None, 0, 8, 0, 1e4, None) == NR_OK
    assert lib.rmsnorm_bwd(BF16, None, None, None, None, None, None, 0, 8, 0, None, 0, None) == NR_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import importlib
    import sys
    monkeypatch.setattr(nr, "_L", None)
    monkeypatch.setattr(nr, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        nr._lib()
