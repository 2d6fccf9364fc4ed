"""Thin Python binding of libnormrope.so (the C ABI in include/normrope.h).

Every function here only marshals arguments: it checks tensor devices,
dtypes and shapes, allocates outputs the caller did not pass, and hands raw
device pointers plus PyTorch's current HIP stream to the C function of the
same name.  All arithmetic happens in the library's HIP kernels; there is no
CPU or PyTorch fallback -- if the library is missing this module raises.

The operations follow "Helios 性能优化全解析" (sections 内核一 FlashNorm and
内核二 FlashRoPE); see include/normrope.h for the exact definitions.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "NormRopeError", "rmsnorm_fwd", "rmsnorm_bwd", "rmsnorm_bwd_noalloc", "layernorm_fwd",
    "layernorm_bwd",
    "rmsnorm_rope_fwd", "rmsnorm_rope_bwd", "layernorm_gelu_fwd", "layernorm_gelu_bwd",
    "rope_interleaved_apply", "rope_table_1d", "rope_table_3d", "nr_bwd_workspace_bytes",
    "nr_status_str", "nr_tune", "nr_norm_n_max", "nr_stream_copy", "nr_stream_mix", "rmsnorm_linear_fwd",
    "rmsnorm_linear_fold_weight", "nr_rmsnorm_linear_workspace_bytes", "layernorm_linear_fwd",
    "nr_layernorm_linear_workspace_bytes",
    "library_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnormrope.so")

NR_F32, NR_BF16, NR_F16 = 0, 1, 2
# rows longer than this take the two-pass backward, whose workspace is
# needed even without column gradients (see rmsnorm_bwd in normrope.h)
_LONG_ROW = 16384
_DT = {torch.float32: NR_F32, torch.bfloat16: NR_BF16, torch.float16: NR_F16}


class NormRopeError(RuntimeError):
    """A non-zero nr_status_t from the library."""

    def __init__(self, fn: str, status: int):
        msg = _lib().nr_status_str(status).decode()
        if status == 6:  # NR_ERR_HIP
            msg += f" (hipError {_lib().nr_last_hip_error()})"
        super().__init__(f"{fn}: {msg} (status {status})")
        self.status = status


_L = None


def library_path() -> str:
    return _LIB_PATH


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                f"{_LIB_PATH} is not built; run `python -m rmsnorm_layernorm_fwd_amd.build` "
                "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
        sig = {
            "rmsnorm_fwd": [i32, vp, vp, vp, vp, i64, i64, f32, i32, vp],
            "rmsnorm_bwd": [i32, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp],
            "rmsnorm_bwd_noalloc": [i32, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp],
            "layernorm_fwd": [i32, vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "layernorm_bwd": [i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, sz, vp],
            "rope_interleaved_apply": [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i32, vp],
            "rmsnorm_rope_fwd": [i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, vp],
            "layernorm_gelu_fwd": [i32, vp, vp, vp, vp, vp, vp, i64, i64, f32, vp],
            "layernorm_gelu_bwd": [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp, sz, vp],
            "rmsnorm_rope_bwd": [i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp, sz, vp],
            "rope_table_1d": [vp, vp, i64, i64, i64, f64, vp],
            "rope_table_3d": [vp, vp, i64, i64, i64, i64, i64, i64, f64, vp],
            "nr_bwd_workspace_bytes": [i64, i64, i32],
            "nr_status_str": [i32],
            "nr_last_hip_error": [],
            "nr_tune": [ctypes.c_char_p, i32],
            "nr_norm_n_max": [i32],
            "nr_stream_copy": [vp, vp, sz, vp],
            "nr_stream_mix": [vp, vp, vp, sz, i32, vp],
            "rmsnorm_linear_fwd": [i32, vp, vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, sz, vp],
            "nr_rmsnorm_linear_workspace_bytes": [i64, i64, i64, i32],
            "rmsnorm_linear_fold_weight": [i32, vp, vp, vp, i64, i64, i32, vp],
            "layernorm_linear_fwd": [i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, vp, sz, vp],
            "nr_layernorm_linear_workspace_bytes": [i64, i64, i64, i32],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.nr_bwd_workspace_bytes.restype = sz
        L.nr_rmsnorm_linear_workspace_bytes.restype = sz
        L.nr_layernorm_linear_workspace_bytes.restype = sz
        L.nr_status_str.restype = ctypes.c_char_p
        L.nr_norm_n_max.restype = i64
        _L = L
    return _L


def _check(fn: str, status: int):
    if status != 0:
        raise NormRopeError(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _run(fn: str, ref: torch.Tensor, *args):
    """Calls library function fn with args plus PyTorch's current stream on
    ref's device, that device being current (the library launches on the
    current device)."""
    with torch.cuda.device(ref.device):
        _check(fn, getattr(_lib(), fn)(*args, _stream(ref)))


def _dev(name: str, t: torch.Tensor, dtype=None, shape=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows_n(x: torch.Tensor):
    n = x.shape[-1]
    return x.numel() // n if n else 0, n


def _dtype_code(x: torch.Tensor) -> int:
    if x.dtype not in _DT:
        raise ValueError(f"unsupported dtype {x.dtype} (fp32, bf16 or fp16)")
    return _DT[x.dtype]


def _workspace(rows, n, ln, ws, device):
    need = nr_bwd_workspace_bytes(rows, n, ln)
    if ws is None:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    _dev("workspace", ws, device=device)
    return ws, ws.numel() * ws.element_size()


# ---------------------------------------------------------------- norms

def rmsnorm_fwd(x, w=None, eps=1e-6, gemma_offset=False, y=None, inv_rms=None, want_stats=True):
    """y = (x * r) * w' per row, r = 1/sqrt(mean(x^2) + eps); returns (y, inv_rms)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("w", w, x.dtype, (n,), device=x.device)
    if y is None:
        y = torch.empty_like(x)
    _dev("y", y, x.dtype, x.shape, device=x.device)
    if inv_rms is None and want_stats:
        inv_rms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    _run("rmsnorm_fwd", x,
         dt, _ptr(x), _ptr(w), _ptr(y), _ptr(inv_rms), rows, n, float(eps),
         int(bool(gemma_offset)))
    return y, inv_rms


def rmsnorm_bwd(dy, x, w, inv_rms, gemma_offset=False, dx=None, want_dw=True, dw=None,
                workspace=None):
    """Backward of rmsnorm_fwd from the cached inv_rms; returns (dx, dw)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("dy", dy, x.dtype, x.shape, device=x.device)
    _dev("w", w, x.dtype, (n,), device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    if dx is None:
        dx = torch.empty_like(x)
    _dev("dx", dx, x.dtype, x.shape, device=x.device)
    if dw is None and want_dw:
        dw = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev("dw", dw, torch.float32, (n,), device=x.device)
    ws, wsb = (None, 0)
    if dw is not None or n > _LONG_ROW:
        ws, wsb = _workspace(rows, n, 0, workspace, x.device)
    _run("rmsnorm_bwd", x,
         dt, _ptr(dy), _ptr(x), _ptr(w), _ptr(inv_rms), _ptr(dx), _ptr(dw), rows, n,
         int(bool(gemma_offset)), _ptr(ws), wsb)
    return dx, dw


def rmsnorm_bwd_noalloc(dy, x, w, inv_rms, dx, dw=None, gemma_offset=False):
    """rmsnorm_bwd with the library's own scratch array instead of a
    workspace: nothing is allocated, here or in the library (dx, and dw when
    wanted, are the caller's).  Calls that may overlap on one GPU race on the
    shared array."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("dy", dy, x.dtype, x.shape, device=x.device)
    _dev("w", w, x.dtype, (n,), device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    _dev("dx", dx, x.dtype, x.shape, device=x.device)
    _dev("dw", dw, torch.float32, (n,), device=x.device)
    _run("rmsnorm_bwd_noalloc", x,
         dt, _ptr(dy), _ptr(x), _ptr(w), _ptr(inv_rms), _ptr(dx), _ptr(dw), rows, n,
         int(bool(gemma_offset)))
    return dx, dw


def layernorm_fwd(x, gamma=None, beta=None, eps=1e-5, y=None, mean=None, rstd=None,
                  want_stats=True):
    """y = (x - mu) r gamma + beta per row; returns (y, mean, rstd)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("gamma", gamma, x.dtype, (n,), device=x.device)
    _dev("beta", beta, x.dtype, (n,), device=x.device)
    if y is None:
        y = torch.empty_like(x)
    _dev("y", y, x.dtype, x.shape, device=x.device)
    if want_stats:
        if mean is None:
            mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("mean", mean, torch.float32, x.shape[:-1], device=x.device)
    _dev("rstd", rstd, torch.float32, x.shape[:-1], device=x.device)
    _run("layernorm_fwd", x,
         dt, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, n,
         float(eps))
    return y, mean, rstd


def layernorm_bwd(dy, x, gamma, mean, rstd, dx=None, want_dgamma=True, want_dbeta=True,
                  dgamma=None, dbeta=None, workspace=None):
    """Backward of layernorm_fwd from the cached mean / rstd; returns (dx, dgamma, dbeta)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("dy", dy, x.dtype, x.shape, device=x.device)
    _dev("gamma", gamma, x.dtype, (n,), device=x.device)
    _dev("mean", mean, torch.float32, x.shape[:-1], device=x.device)
    _dev("rstd", rstd, torch.float32, x.shape[:-1], device=x.device)
    if dx is None:
        dx = torch.empty_like(x)
    _dev("dx", dx, x.dtype, x.shape, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(n, dtype=torch.float32, device=x.device)
    if dbeta is None and want_dbeta:
        dbeta = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev("dgamma", dgamma, torch.float32, (n,), device=x.device)
    _dev("dbeta", dbeta, torch.float32, (n,), device=x.device)
    ws, wsb = (None, 0)
    if dgamma is not None or dbeta is not None or n > _LONG_ROW:
        ws, wsb = _workspace(rows, n, 1, workspace, x.device)
    _run("layernorm_bwd", x,
         dt, _ptr(dy), _ptr(x), _ptr(gamma), _ptr(mean), _ptr(rstd), _ptr(dx), _ptr(dgamma),
         _ptr(dbeta), rows, n, _ptr(ws), wsb)
    return dx, dgamma, dbeta


# ---------------------------------------------------------------- fused LayerNorm + GeLU

def layernorm_gelu_fwd(x, gamma=None, beta=None, eps=1e-5, y=None, mean=None, rstd=None,
                       want_stats=True):
    """y = gelu_tanh((x - mu) r gamma + beta) in one pass; returns (y, mean, rstd)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("gamma", gamma, x.dtype, (n,), device=x.device)
    _dev("beta", beta, x.dtype, (n,), device=x.device)
    if y is None:
        y = torch.empty_like(x)
    _dev("y", y, x.dtype, x.shape, device=x.device)
    if want_stats:
        if mean is None:
            mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("mean", mean, torch.float32, x.shape[:-1], device=x.device)
    _dev("rstd", rstd, torch.float32, x.shape[:-1], device=x.device)
    _run("layernorm_gelu_fwd", x,
         dt, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), _ptr(mean), _ptr(rstd), rows, n,
         float(eps))
    return y, mean, rstd


def layernorm_gelu_bwd(dout, x, gamma, beta, mean, rstd, dx=None, want_dgamma=True,
                       want_dbeta=True, dgamma=None, dbeta=None, workspace=None):
    """Backward of layernorm_gelu_fwd; returns (dx, dgamma, dbeta)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rows_n(x)
    _dev("dout", dout, x.dtype, x.shape, device=x.device)
    _dev("gamma", gamma, x.dtype, (n,), device=x.device)
    _dev("beta", beta, x.dtype, (n,), device=x.device)
    _dev("mean", mean, torch.float32, x.shape[:-1], device=x.device)
    _dev("rstd", rstd, torch.float32, x.shape[:-1], device=x.device)
    if dx is None:
        dx = torch.empty_like(x)
    _dev("dx", dx, x.dtype, x.shape, device=x.device)
    if dgamma is None and want_dgamma:
        dgamma = torch.empty(n, dtype=torch.float32, device=x.device)
    if dbeta is None and want_dbeta:
        dbeta = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev("dgamma", dgamma, torch.float32, (n,), device=x.device)
    _dev("dbeta", dbeta, torch.float32, (n,), device=x.device)
    ws, wsb = (None, 0)
    if dgamma is not None or dbeta is not None or n > _LONG_ROW:
        ws, wsb = _workspace(rows, n, 1, workspace, x.device)
    _run("layernorm_gelu_bwd", x,
         dt, _ptr(dout), _ptr(x), _ptr(gamma), _ptr(beta), _ptr(mean), _ptr(rstd), _ptr(dx),
         _ptr(dgamma), _ptr(dbeta), rows, n, _ptr(ws), wsb)
    return dx, dgamma, dbeta


# ---------------------------------------------------------------- fused RMSNorm + RoPE

def _rope_rows(x, cos_tab, sin_tab, head_dim, rows_per_token):
    rows, n = _rows_n(x)
    if head_dim <= 0 or n % head_dim:
        raise ValueError("the row length must be a whole number of head vectors")
    tokens = -(-rows // rows_per_token) if rows else 0
    _dev("cos_tab", cos_tab, torch.float32, (tokens, head_dim // 2), device=x.device)
    _dev("sin_tab", sin_tab, torch.float32, (tokens, head_dim // 2), device=x.device)
    return rows, n


def rmsnorm_rope_fwd(x, w, cos_tab, sin_tab, head_dim, rows_per_token=1, eps=1e-6,
                     gemma_offset=False, y=None, inv_rms=None, want_stats=True):
    """rope(rmsnorm(x)) in one pass; rows of n = heads x head_dim; returns (y, inv_rms)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rope_rows(x, cos_tab, sin_tab, head_dim, rows_per_token)
    _dev("w", w, x.dtype, (n,), device=x.device)
    if y is None:
        y = torch.empty_like(x)
    _dev("y", y, x.dtype, x.shape, device=x.device)
    if inv_rms is None and want_stats:
        inv_rms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    _run("rmsnorm_rope_fwd", x,
         dt, _ptr(x), _ptr(w), _ptr(y), _ptr(inv_rms), _ptr(cos_tab), _ptr(sin_tab), rows, n,
         head_dim, rows_per_token, float(eps), int(bool(gemma_offset)))
    return y, inv_rms


def rmsnorm_rope_bwd(dout, x, w, inv_rms, cos_tab, sin_tab, head_dim, rows_per_token=1,
                     gemma_offset=False, dx=None, want_dw=True, dw=None, workspace=None):
    """Backward of rmsnorm_rope_fwd; returns (dx, dw)."""
    _dev("x", x)
    dt = _dtype_code(x)
    rows, n = _rope_rows(x, cos_tab, sin_tab, head_dim, rows_per_token)
    _dev("dout", dout, x.dtype, x.shape, device=x.device)
    _dev("w", w, x.dtype, (n,), device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    if dx is None:
        dx = torch.empty_like(x)
    _dev("dx", dx, x.dtype, x.shape, device=x.device)
    if dw is None and want_dw:
        dw = torch.empty(n, dtype=torch.float32, device=x.device)
    _dev("dw", dw, torch.float32, (n,), device=x.device)
    ws, wsb = (None, 0)
    if dw is not None or n > _LONG_ROW:
        ws, wsb = _workspace(rows, n, 2, workspace, x.device)
    _run("rmsnorm_rope_bwd", x,
         dt, _ptr(dout), _ptr(x), _ptr(w), _ptr(inv_rms), _ptr(cos_tab), _ptr(sin_tab), _ptr(dx),
         _ptr(dw), rows, n, head_dim, rows_per_token, int(bool(gemma_offset)), _ptr(ws), wsb)
    return dx, dw


# ---------------------------------------------------------------- RoPE

def rope_interleaved_apply(x, cos_tab, sin_tab, inverse=False):
    """Rotate interleaved pairs of x [B, T, H, D] in place (strides taken from x)."""
    if x.dim() != 4:
        raise ValueError("x must be [batch, tokens, heads, head_dim]")
    if x.device.type != "cuda" or x.stride(3) != 1:
        raise ValueError("x must be a GPU tensor with a contiguous last axis")
    dt = _dtype_code(x)
    b, t, h, d = x.shape
    _dev("cos_tab", cos_tab, torch.float32, (t, d // 2), device=x.device)
    _dev("sin_tab", sin_tab, torch.float32, (t, d // 2), device=x.device)
    _run("rope_interleaved_apply", x,
         dt, _ptr(x), _ptr(cos_tab), _ptr(sin_tab), b, t, h, d, x.stride(0), x.stride(1),
         x.stride(2), int(bool(inverse)))
    return x


def rope_table_1d(tokens, head_dim, pos0=0, theta=10000.0, device="cuda"):
    """fp32 cos/sin tables [tokens, head_dim/2] for positions pos0.."""
    c = torch.empty((tokens, head_dim // 2), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _run("rope_table_1d", c, _ptr(c), _ptr(s), tokens, head_dim, pos0, float(theta))
    return c, s


def rope_table_3d(grid, pairs, theta=10000.0, device="cuda"):
    """fp32 cos/sin tables [F*H*W, sum(pairs)] for a frames x height x width grid."""
    f, h, w = grid
    pt, ph, pw = pairs
    c = torch.empty((f * h * w, pt + ph + pw), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _run("rope_table_3d", c, _ptr(c), _ptr(s), f, h, w, pt, ph, pw, float(theta))
    return c, s


# ---------------------------------------------------------------- RMSNorm -> linear

def rmsnorm_linear_fwd(x, w_norm, W, eps=1e-6, gemma_offset=False, out=None, inv_rms=None,
                       want_stats=True, workspace=None):
    """out = rmsnorm(x, w_norm) @ W.T with the norm folded into the GEMM
    (bf16; W [N, K] as a linear layer stores it); returns (out, inv_rms).
    The folded weight goes to `workspace` (allocated here when None and the
    call needs one)."""
    _dev("x", x, torch.bfloat16)
    rows, k = _rows_n(x)
    _dev("W", W, torch.bfloat16, device=x.device)
    if W.dim() != 2 or W.shape[1] != k:
        raise ValueError(f"W must be [N, {k}]")
    n = W.shape[0]
    _dev("w_norm", w_norm, torch.bfloat16, (k,), device=x.device)
    if out is None:
        out = torch.empty(x.shape[:-1] + (n,), dtype=torch.bfloat16, device=x.device)
    _dev("out", out, torch.bfloat16, x.shape[:-1] + (n,), device=x.device)
    if inv_rms is None and want_stats:
        inv_rms = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("inv_rms", inv_rms, torch.float32, x.shape[:-1], device=x.device)
    wsb = nr_rmsnorm_linear_workspace_bytes(rows, n, k, w_norm is not None)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _dev("workspace", workspace, device=x.device)
    _run("rmsnorm_linear_fwd", x,
         NR_BF16, _ptr(x), _ptr(w_norm), _ptr(W), _ptr(out), _ptr(inv_rms), rows, n, k, float(eps),
         int(bool(gemma_offset)), _ptr(workspace),
         0 if workspace is None else workspace.numel() * workspace.element_size())
    return out, inv_rms


def rmsnorm_linear_fold_weight(w_norm, W, gemma_offset=False, out=None):
    """W_folded = bf16(W * w'): the weight rmsnorm_linear_fwd multiplies by,
    for calls with w_norm=None (bit-identical output, no workspace)."""
    _dev("W", W, torch.bfloat16)
    if W.dim() != 2:
        raise ValueError("W must be [N, K]")
    n, k = W.shape
    _dev("w_norm", w_norm, torch.bfloat16, (k,), device=W.device)
    if out is None:
        out = torch.empty_like(W)
    _dev("W_folded", out, torch.bfloat16, (n, k), device=W.device)
    _run("rmsnorm_linear_fold_weight", W,
         NR_BF16, _ptr(w_norm), _ptr(W), _ptr(out), n, k, int(bool(gemma_offset)))
    return out


def layernorm_linear_fwd(x, gamma, beta, W, eps=1e-5, out=None, mean=None, rstd=None,
                         want_stats=True, workspace=None):
    """out = layernorm(x, gamma, beta) @ W.T with the norm folded into the
    GEMM (bf16; W [N, K] as a linear layer stores it, N % 256 == 0);
    returns (out, mean, rstd)."""
    _dev("x", x, torch.bfloat16)
    rows, k = _rows_n(x)
    _dev("W", W, torch.bfloat16, device=x.device)
    if W.dim() != 2 or W.shape[1] != k:
        raise ValueError(f"W must be [N, {k}]")
    n = W.shape[0]
    _dev("gamma", gamma, torch.bfloat16, (k,), device=x.device)
    _dev("beta", beta, torch.bfloat16, (k,), device=x.device)
    if out is None:
        out = torch.empty(x.shape[:-1] + (n,), dtype=torch.bfloat16, device=x.device)
    _dev("out", out, torch.bfloat16, x.shape[:-1] + (n,), device=x.device)
    if want_stats:
        if mean is None:
            mean = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
        if rstd is None:
            rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _dev("mean", mean, torch.float32, x.shape[:-1], device=x.device)
    _dev("rstd", rstd, torch.float32, x.shape[:-1], device=x.device)
    wsb = nr_layernorm_linear_workspace_bytes(rows, n, k, gamma is not None)
    if workspace is None and wsb > 0:
        workspace = torch.empty(wsb, dtype=torch.uint8, device=x.device)
    _dev("workspace", workspace, device=x.device)
    _run("layernorm_linear_fwd", x,
         NR_BF16, _ptr(x), _ptr(gamma), _ptr(beta), _ptr(W), _ptr(out), _ptr(mean), _ptr(rstd),
         rows, n, k, float(eps), _ptr(workspace),
         0 if workspace is None else workspace.numel() * workspace.element_size())
    return out, mean, rstd


def nr_layernorm_linear_workspace_bytes(m, n, k, has_gamma) -> int:
    return int(_lib().nr_layernorm_linear_workspace_bytes(m, n, k, int(bool(has_gamma))))


def nr_rmsnorm_linear_workspace_bytes(m, n, k, has_weight) -> int:
    return int(_lib().nr_rmsnorm_linear_workspace_bytes(m, n, k, int(bool(has_weight))))


# ---------------------------------------------------------------- helpers

def nr_bwd_workspace_bytes(rows, n, op) -> int:
    """op: 0 rmsnorm_bwd, 1 layernorm_bwd or layernorm_gelu_bwd, 2 rmsnorm_rope_bwd."""
    return int(_lib().nr_bwd_workspace_bytes(rows, n, int(op)))


def nr_stream_copy(src: torch.Tensor, dst: torch.Tensor):
    """Measurement aid: copy src's bytes into dst with the row kernels'
    streaming access pattern (the practical HBM ceiling)."""
    _dev("src", src)
    _dev("dst", dst, device=src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or src.device != dst.device:
        raise ValueError("nr_stream_copy: src and dst must have the same size and device")
    _run("nr_stream_copy", src, _ptr(src), _ptr(dst), nbytes)


def nr_stream_mix(a: torch.Tensor, b: torch.Tensor, dst: torch.Tensor, write: bool = True):
    """Measurement aid: read a and b (and write a ^ b to dst when `write`)
    with the same access pattern as nr_stream_copy."""
    _dev("a", a)
    _dev("b", b, device=a.device)
    _dev("dst", dst, device=a.device)
    nbytes = a.numel() * a.element_size()
    if any(t.numel() * t.element_size() != nbytes for t in (b, dst)):
        raise ValueError("nr_stream_mix: a, b and dst must have the same size")
    _run("nr_stream_mix", a, _ptr(a), _ptr(b), _ptr(dst), nbytes, int(bool(write)))


def nr_status_str(status: int) -> str:
    return _lib().nr_status_str(status).decode()


def nr_tune(key: str, value: int):
    _check("nr_tune", _lib().nr_tune(key.encode(), int(value)))


def nr_norm_n_max(dtype) -> int:
    return int(_lib().nr_norm_n_max(_DT[dtype]))
