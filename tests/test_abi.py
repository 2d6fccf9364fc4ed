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
    expected = {"rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_noalloc", "layernorm_fwd", "layernorm_bwd",
                "rmsnorm_rope_fwd", "rmsnorm_rope_bwd", "layernorm_gelu_fwd", "layernorm_gelu_bwd",
                "rope_interleaved_apply", "rope_table_1d", "rope_table_3d",
                "nr_bwd_workspace_bytes", "nr_status_str", "nr_last_hip_error", "nr_tune",
                "nr_norm_n_max", "nr_stream_copy", "nr_stream_mix", "rmsnorm_linear_fwd",
                "rmsnorm_linear_fold_weight", "nr_rmsnorm_linear_workspace_bytes",
                "layernorm_linear_fwd", "nr_layernorm_linear_workspace_bytes"}
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
    # narrow rows (few waves a row, counted for 16-bit rows): up to 256 x
    # floor(10 / W) workgroups, at most 4 per CU -- LayerNorm from 5 waves a
    # row down (2560: W = 5, two per CU), RMSNorm from 4 (2048: W = 4, two;
    # 1280: W = 3, three); RMSNorm at 2560 keeps one, the RoPE one is unchanged
    assert nr.nr_bwd_workspace_bytes(65536, 2560, 1) == 2 * 512 * 2560 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 2560, 0) == 256 * 2560 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 2048, 0) == 512 * 2048 * 4
    # (768 allowed; 86 rows each, so 763 with none empty)
    assert nr.nr_bwd_workspace_bytes(65536, 1280, 0) == 763 * 1280 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 1280, 1) == 2 * 763 * 1280 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 512, 1) == 2 * 1024 * 512 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 1280, 2) == 512 * 1280 * 4
    assert nr.nr_bwd_workspace_bytes(15000, 1280, 0) == 750 * 1280 * 4  # 20 rows each
    # rows of at most 32 chunks (a per-head norm) take up to eight a CU
    assert nr.nr_bwd_workspace_bytes(65536, 256, 0) == 2048 * 256 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 128, 1) == 2 * 2048 * 128 * 4
    assert nr.nr_bwd_workspace_bytes(65536, 264, 0) == 1024 * 264 * 4  # 33 chunks
    # RMSNorm -> RoPE on such rows (per-head): up to five a CU
    assert nr.nr_bwd_workspace_bytes(2621440, 128, 2) == 1280 * 128 * 4
    assert nr.nr_bwd_workspace_bytes(4000, 256, 2) == 500 * 256 * 4  # 8 rows each
    assert nr.nr_bwd_workspace_bytes(65536, 264, 2) == 512 * 264 * 4
    assert nr.nr_bwd_workspace_bytes(64, 8, 3) == 0
    # rows of more than 16384 elements (two passes): ceil(rows / 16) partial
    # rows, at most 256 / S where S = ceil(n / 4096) column slices of a 2-byte
    # row (the largest count of the storage types), then two fp32 terms per row
    assert nr.nr_bwd_workspace_bytes(100, 20000, 1) == 7 * 20000 * 4 * 2 + 100 * 8
    assert nr.nr_bwd_workspace_bytes(4096, 32768, 2) == 32 * 32768 * 4 + 4096 * 8
    assert nr.nr_bwd_workspace_bytes(100, 40000, 0) == 7 * 40000 * 4 + 100 * 8
    # plain RMSNorm of 16385..32768 elements: one pass for aligned 16-bit rows
    # (the short-row partial rows), two for the others; the larger size
    assert nr.nr_bwd_workspace_bytes(100, 20000, 0) == 100 * 20000 * 4  # a row a workgroup
    assert nr.nr_bwd_workspace_bytes(8192, 20480, 0) == 256 * 20480 * 4
    assert nr.nr_bwd_workspace_bytes(512, 32768, 0) == 256 * 32768 * 4
    assert nr.nr_bwd_workspace_bytes(300, 32768, 0) == 150 * 32768 * 4  # 2 rows each
    assert nr.nr_bwd_workspace_bytes(1, 32768, 0) == 32768 * 4 + 8  # the two-pass size
    assert nr.nr_bwd_workspace_bytes(4096, 65536, 1) == 2 * 16 * 65536 * 4 + 4096 * 8
    assert nr.nr_bwd_workspace_bytes(160, 65536, 1) == 2 * 10 * 65536 * 4 + 160 * 8


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
    # the two tables of a builder may not share bytes
    assert L.rope_table_1d(FAKE, FAKE + 32, 4, 8, 0, 1e4, None) == NR_ERR_ALIAS  # 64-byte tables
    # RoPE: x (rewritten in place) may not overlap its tables
    assert L.rope_interleaved_apply(F32, FAKE, FAKE + 64, 0x90000, 1, 4, 2, 8, 64, 16, 8, 0, None) == NR_ERR_ALIAS
    assert L.rope_interleaved_apply(F32, FAKE, 0x90000, FAKE + 200, 1, 4, 2, 8, 64, 16, 8, 0, None) == NR_ERR_ALIAS
    assert L.rope_table_3d(FAKE, FAKE + 64, 2, 3, 4, 2, 2, 2, 1e4, None) == NR_ERR_ALIAS
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
    # (64 x 256 fp32 rows: dy at FAKE, x, dx 64 KiB each; statistics, dw,
    # dbeta and the workspace in ranges of their own)
    R, MU, DW, DB, WS = 0xC0000, 0xC8000, 0xD0000, 0xD8000, 0xE0000
    need = nr.nr_bwd_workspace_bytes(64, 256, 0)
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, DW, 64, 256, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, DW, 64, 256, 0, WS, need - 4, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, DW, 64, 256, 0, WS + 4, need, None) == NR_ERR_WORKSPACE
    need_ln = nr.nr_bwd_workspace_bytes(64, 256, 1)
    assert L.layernorm_bwd(F32, FAKE, 0x90000, None, MU, R, 0xA0000, None, DB, 64, 256, WS, need_ln - 1, None) == NR_ERR_WORKSPACE
    # every other output and the workspace share no byte with any operand:
    # dx over the statistics or the weight, a column gradient over dy, over
    # the workspace or over the other one, the workspace over x
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, 0xA0000 + 256, 0xA0000, DW, 64, 256, 0, WS, need, None) == NR_ERR_ALIAS
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, 0xA0000 + 512, R, 0xA0000, DW, 64, 256, 0, WS, need, None) == NR_ERR_ALIAS
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, FAKE + 64, 64, 256, 0, WS, need, None) == NR_ERR_ALIAS
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, WS + 16, 64, 256, 0, WS, need, None) == NR_ERR_ALIAS
    assert L.rmsnorm_bwd(F32, FAKE, 0x90000, None, R, 0xA0000, DW, 64, 256, 0, 0x90000 + 1024, need, None) == NR_ERR_ALIAS
    assert L.layernorm_bwd(F32, FAKE, 0x90000, None, MU, R, 0xA0000, DB, DB + 512, 64, 256, WS, need_ln, None) == NR_ERR_ALIAS
    # the forward: y over the weight, the statistics over x or over each other
    assert L.rmsnorm_fwd(F32, FAKE, 0xA0000 + 1024, 0xA0000, None, 64, 256, 1e-6, 0, None) == NR_ERR_ALIAS
    assert L.rmsnorm_fwd(F32, FAKE, None, 0xA0000, FAKE + 4, 64, 256, 1e-6, 0, None) == NR_ERR_ALIAS
    assert L.layernorm_fwd(F32, FAKE, None, None, 0xA0000, R, R + 128, 64, 256, 1e-5, None) == NR_ERR_ALIAS
    assert L.layernorm_gelu_fwd(F32, FAKE, 0xA0000 + 64, None, 0xA0000, R, MU, 64, 256, 1e-5, None) == NR_ERR_ALIAS
    # grids beyond the hardware's 2^31 - 1 workgroups are refused, not truncated
    FAR = 1 << 40
    assert L.rmsnorm_fwd(BF16, FAKE, None, FAR, None, 1 << 34, 1, 1e-6, 0, None) == NR_ERR_SHAPE
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
    # LayerNorm -> linear: bf16, N % 256, K % 64, pointers, alignment,
    # workspace size / alignment / overlap
    ll = L.layernorm_linear_fwd
    lw = nr.nr_layernorm_linear_workspace_bytes(4, 256, 64, True)
    assert lw == 2 * 256 + 2 * 1024 + 256 * 64 * 2
    assert nr.nr_layernorm_linear_workspace_bytes(4, 256, 64, False) == 2 * 256 + 2 * 1024
    WS = 1 << 34
    args = lambda m, n, k: (m, n, k, 1e-5)
    assert ll(F32, XA, None, None, WA, OA, None, None, *args(4, 256, 64), WS, lw, None) == NR_ERR_DTYPE
    assert ll(BF16, XA, None, None, WA, OA, None, None, *args(4, 128, 64), WS, lw, None) == NR_ERR_SHAPE
    assert ll(BF16, XA, None, None, WA, OA, None, None, *args(4, 256, 72), WS, lw, None) == NR_ERR_SHAPE
    assert ll(BF16, None, None, None, WA, OA, None, None, *args(4, 256, 64), WS, lw, None) == NR_ERR_NULLPTR
    assert ll(BF16, XA, XA + 2, None, WA, OA, None, None, *args(4, 256, 64), WS, lw, None) == NR_ERR_SHAPE
    assert ll(BF16, XA, None, None, WA, XA + 64, None, None, *args(4, 256, 64), WS, lw, None) == NR_ERR_ALIAS
    assert ll(BF16, XA, FAKE, None, WA, OA, None, None, *args(4, 256, 64), None, 0, None) == NR_ERR_WORKSPACE
    assert ll(BF16, XA, FAKE, None, WA, OA, None, None, *args(4, 256, 64), WS, lw - 16, None) == NR_ERR_WORKSPACE
    assert ll(BF16, XA, FAKE, None, WA, OA, None, None, *args(4, 256, 64), WS + 8, lw, None) == NR_ERR_WORKSPACE
    assert ll(BF16, XA, FAKE, None, WA, OA, None, None, *args(4, 256, 64), WA + 512, lw, None) == NR_ERR_ALIAS
    assert ll(BF16, None, None, None, None, None, None, None, *args(0, 256, 64), None, 0, None) == NR_OK
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
    assert L.nr_stream_mix(FAKE, None, 0x90000, 64, 1, None) == NR_ERR_NULLPTR
    assert L.nr_stream_mix(FAKE, 0x80000, 0x90000, 60, 1, None) == NR_ERR_SHAPE
    assert L.nr_stream_mix(FAKE, 0x80000, FAKE + 32, 64, 0, None) == NR_ERR_ALIAS
    assert L.nr_stream_mix(FAKE, 0x80000, 0x80000, 64, 1, None) == NR_ERR_ALIAS
    assert L.nr_stream_mix(None, None, None, 0, 1, None) == NR_OK
    # the no-allocation backward: a shape whose workspace exceeds its 32 MiB
    # scratch array (2^22 rows of 65536: 4 MiB of partial rows and 32 MiB of
    # row terms) is refused before anything else; a shape needing no scratch
    # (no dw, short rows) goes straight to rmsnorm_bwd's checks
    X = 1 << 24
    assert nr.nr_bwd_workspace_bytes(1 << 22, 65536, 0) > 32 << 20
    assert nr.nr_bwd_workspace_bytes(1 << 20, 32768, 0) <= 32 << 20  # the one pass fits
    assert L.rmsnorm_bwd_noalloc(BF16, FAKE, X, None, FAKE, 1 << 30, FAKE, 1 << 22, 65536, 0,
                                 None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd_noalloc(7, FAKE, X, None, FAKE, 1 << 25, None, 4, 8, 0, None) == NR_ERR_DTYPE
    # rows that take two passes need the workspace even without a column
    # gradient: bf16 past 32768 elements, or past 16384 when not a multiple
    # of 8 (element-wise), fp32 past 16384
    X2, DX2, WS2, R2 = 1 << 24, 1 << 25, 1 << 26, 1 << 27
    assert L.rmsnorm_bwd(BF16, FAKE, X2, None, R2, DX2, None, 4, 40000, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(BF16, FAKE, X2, None, R2, DX2, None, 4, 20001, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.rmsnorm_bwd(F32, FAKE, X2, None, R2, DX2, None, 4, 20000, 0, None, 0, None) == NR_ERR_WORKSPACE
    assert L.layernorm_bwd(F32, FAKE, X2, None, R2 + 4096, R2, DX2, None, None, 4, 20000, WS2, 31, None) == NR_ERR_WORKSPACE
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


def test_rope_rejects_overlapping_vectors(lib):
    """Distinct (batch, token, head) vectors of the in-place rotation may not
    share elements: broadcast (stride 0) axes and strides shorter than the
    block inside them are refused before anything is queued.  Packed,
    padded and transposed layouts pass the check; a null table then stops
    them at the null-pointer check, so nothing is launched."""
    L = lib
    A = NR_ERR_ALIAS
    ra = L.rope_interleaved_apply
    # (batch, tokens, heads, head_dim, stride_batch, stride_token, stride_head)
    overlapping = [
        (1, 4, 2, 8, 64, 0, 8),      # tokens broadcast (expand) over one vector
        (2, 4, 2, 8, 0, 16, 8),      # batch broadcast
        (1, 4, 2, 8, 64, 8, 8),      # token stride shorter than a token's two heads
        (1, 4, 3, 8, 64, 16, 8),     # three heads in a 16-element token stride
        (2, 4, 2, 8, 32, 16, 8),     # batch stride shorter than its 4 tokens x 16
        (1, 4, 2, 8, 64, 2, 8),      # token stride inside a head vector
        (1, 4, 2, 8, 64, 16, 4),     # heads overlap (stride_head < head_dim)
        (1, 4, 2, 8, 64, 8, 16),     # [H, T]: the second head starts inside token 2's vector
    ]
    for shp in overlapping:
        assert ra(BF16, FAKE, FAKE, FAKE, *shp, 0, None) == A, shp
    disjoint = [
        (1, 4, 2, 8, 64, 16, 8),     # packed
        (2, 4, 2, 8, 64, 16, 8),     # packed batches
        (1, 4, 2, 8, 128, 24, 8),    # padded tokens
        (2, 4, 2, 8, 64, 8, 32),     # [B, H, T, D]: heads outermost within a batch
        (1, 1, 2, 8, 0, 0, 8),       # size-1 axes may have any stride
        (3, 4, 1, 8, 32, 8, 0),      # one head: its stride is irrelevant
    ]
    for shp in disjoint:
        # passes the overlap check and stops at the (later) null-pointer check
        assert ra(BF16, FAKE, None, FAKE, *shp, 0, None) == NR_ERR_NULLPTR, shp


def test_binding_checks_stat_shapes_before_launch(monkeypatch):
    """A caller-supplied statistics buffer of the wrong shape is refused by
    the binding before the library is called (a short buffer would let the
    kernels' per-row statistics stores run past it).  The tensors are CPU
    tensors posing as GPU tensors; the library call itself is replaced by a
    trap, so nothing runs on a device."""
    import torch

    class Posing(torch.Tensor):
        @property
        def device(self):
            return torch.device("cuda", 0)

    def fake(t):
        return torch.Tensor._make_subclass(Posing, t)

    def trap(*a, **k):
        raise AssertionError("library called despite a bad statistics buffer")

    monkeypatch.setattr(nr, "_run", trap)
    x = fake(torch.zeros(6, 16, dtype=torch.bfloat16))
    y = fake(torch.zeros(6, 16, dtype=torch.bfloat16))
    w = fake(torch.zeros(16, dtype=torch.bfloat16))
    short = fake(torch.zeros(5, dtype=torch.float32))
    ok = fake(torch.zeros(6, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        nr.rmsnorm_fwd(x, w, y=y, inv_rms=short)
    with pytest.raises(ValueError, match="shape"):
        nr.layernorm_fwd(x, w, w, y=y, mean=short, rstd=ok)
    with pytest.raises(ValueError, match="shape"):
        nr.layernorm_fwd(x, w, w, y=y, mean=ok, rstd=short)
    with pytest.raises(ValueError, match="shape"):
        nr.layernorm_gelu_fwd(x, w, w, y=y, mean=ok, rstd=short)
    ct = fake(torch.zeros(6, 4, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        nr.rmsnorm_rope_fwd(x, w, ct, ct, 8, 1, y=y, inv_rms=short)
    xl = fake(torch.zeros(6, 64, dtype=torch.bfloat16))
    Wl = fake(torch.zeros(128, 64, dtype=torch.bfloat16))
    ol = fake(torch.zeros(6, 128, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        nr.rmsnorm_linear_fwd(xl, None, Wl, out=ol, inv_rms=short)
    # the right shapes reach the (trapped) library call
    with pytest.raises(AssertionError, match="library called"):
        nr.rmsnorm_fwd(x, w, y=y, inv_rms=ok)
