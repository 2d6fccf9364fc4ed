"""fp64 CPU oracle for the norm and RoPE operators (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check
and by the benchmark's CPU-baseline leg, never by the product library.  It
shares no code with the HIP path.  Every function takes the exact input
tensors the GPU consumed (fp32 / bf16 / fp64, CPU) and returns float64 numpy
arrays that are never rounded to the storage dtype.  Storage types: fp64,
fp32, bf16 and IEEE fp16, widened exactly.

The arithmetic lives in oracle.c; each function there cites the page section
it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_DT = {torch.float64: 0, torch.float32: 1, torch.bfloat16: 2, torch.float16: 3}


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (IEEE double: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(build())
        vp, i32, i64, f64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_rmsnorm_fwd.argtypes = [vp, i32, vp, i32, i32, i64, i64, f64, vp, vp]
        L.oracle_rmsnorm_bwd.argtypes = [vp, vp, i32, vp, i32, i32, i64, i64, f64, vp, vp]
        L.oracle_layernorm_fwd.argtypes = [vp, i32, vp, vp, i32, i64, i64, f64, vp, vp, vp]
        L.oracle_layernorm_bwd.argtypes = [vp, vp, i32, vp, i32, i64, i64, f64, vp, vp, vp]
        L.oracle_rope_angles_1d.argtypes = [i64, i64, i64, f64, vp]
        L.oracle_rope_angles_3d.argtypes = [i64, i64, i64, i64, i64, i64, f64, vp]
        L.oracle_rope_apply.argtypes = [vp, i32, i64, i64, i64, i64, vp, i32, vp]
        L.oracle_layernorm_gelu_fwd.argtypes = [vp, i32, vp, vp, i32, i64, i64, f64, vp, vp, vp]
        L.oracle_layernorm_gelu_bwd.argtypes = [vp, vp, i32, vp, vp, i32, i64, i64, f64, vp, vp, vp]
        L.oracle_gelu_tanh.argtypes = [f64]
        L.oracle_gelu_tanh_grad.argtypes = [f64]
        L.oracle_widen.argtypes = [vp, i32, i64, vp]
        L.oracle_widen.restype = None
        L.oracle_max_threads.argtypes = []
        L.oracle_max_threads.restype = i32
        L.oracle_gelu_tanh.restype = f64
        L.oracle_gelu_tanh_grad.restype = f64
        for f in ("oracle_rmsnorm_fwd", "oracle_rmsnorm_bwd", "oracle_layernorm_fwd",
                  "oracle_layernorm_bwd", "oracle_rope_angles_1d", "oracle_rope_angles_3d",
                  "oracle_rope_apply", "oracle_layernorm_gelu_fwd", "oracle_layernorm_gelu_bwd"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


class _In:
    """Keeps a contiguous CPU copy alive and exposes (pointer, dtype code)."""

    def __init__(self, t):
        if t is None:
            self.t, self.p, self.dt = None, None, 0
            return
        if isinstance(t, np.ndarray):
            t = torch.from_numpy(t)
        t = t.detach().cpu().contiguous()
        if t.dtype not in _DT:
            raise TypeError(f"oracle: unsupported dtype {t.dtype}")
        self.t, self.p, self.dt = t, t.data_ptr(), _DT[t.dtype]


def _out(*shape):
    return np.zeros(shape, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _rows_n(x):
    n = x.shape[-1]
    return (x.numel() // n if n else 0), n


def rmsnorm_fwd(x, w=None, eps=1e-6, gemma=False):
    """D1 -> (y [rows, n], inv_rms [rows]) in float64."""
    X, W = _In(x), _In(w)
    m, n = _rows_n(X.t)
    y, r = _out(m, n), _out(m)
    lib().oracle_rmsnorm_fwd(X.p, X.dt, W.p, W.dt, int(gemma), m, n, float(eps), _ptr(y), _ptr(r))
    return y, r


def rmsnorm_bwd(dy, x, w=None, eps=1e-6, gemma=False, want_dx=True, want_dw=True):
    """D2 -> (dx [rows, n] or None, dw [n] or None) in float64."""
    DY, X, W = _In(dy), _In(x), _In(w)
    if DY.dt != X.dt:
        raise TypeError("oracle: dy and x must share a dtype")
    m, n = _rows_n(X.t)
    dx = _out(m, n) if want_dx else None
    dw = _out(n) if want_dw else None
    lib().oracle_rmsnorm_bwd(DY.p, X.p, X.dt, W.p, W.dt, int(gemma), m, n, float(eps),
                             _ptr(dx), _ptr(dw))
    return dx, dw


def layernorm_fwd(x, gamma=None, beta=None, eps=1e-5):
    """D3 -> (y, mean, rstd) in float64."""
    X, G, B = _In(x), _In(gamma), _In(beta)
    if G.t is not None and B.t is not None and G.dt != B.dt:
        raise TypeError("oracle: gamma and beta must share a dtype")
    m, n = _rows_n(X.t)
    y, mu, r = _out(m, n), _out(m), _out(m)
    lib().oracle_layernorm_fwd(X.p, X.dt, G.p, B.p, G.dt if G.t is not None else B.dt,
                               m, n, float(eps), _ptr(y), _ptr(mu), _ptr(r))
    return y, mu, r


def layernorm_bwd(dy, x, gamma=None, eps=1e-5, want_dx=True, want_dw=True):
    """D4 -> (dx, dgamma, dbeta) in float64."""
    DY, X, G = _In(dy), _In(x), _In(gamma)
    if DY.dt != X.dt:
        raise TypeError("oracle: dy and x must share a dtype")
    m, n = _rows_n(X.t)
    dx = _out(m, n) if want_dx else None
    dg = _out(n) if want_dw else None
    db = _out(n) if want_dw else None
    lib().oracle_layernorm_bwd(DY.p, X.p, X.dt, G.p, G.dt, m, n, float(eps),
                               _ptr(dx), _ptr(dg), _ptr(db))
    return dx, dg, db


def rope_angles_1d(tokens, head_dim, pos0=0, theta=10000.0):
    """D5 (1-D) -> angle [tokens, head_dim/2] float64."""
    a = _out(tokens, head_dim // 2)
    lib().oracle_rope_angles_1d(tokens, head_dim, pos0, float(theta), _ptr(a))
    return a


def rope_angles_3d(grid, pairs, theta=10000.0):
    """D5 (3-D) -> angle [F*H*W, sum(pairs)] float64."""
    f, h, w = grid
    pt, ph, pw = pairs
    a = _out(f * h * w, pt + ph + pw)
    lib().oracle_rope_angles_3d(f, h, w, pt, ph, pw, float(theta), _ptr(a))
    return a


def rope_angles(spec: dict, tokens: int, head_dim: int):
    """Angles for a table spec as produced by ``workloads.rope_inputs``."""
    if spec["kind"] == "1d":
        return rope_angles_1d(tokens, head_dim, spec.get("pos0", 0), spec["theta"])
    f, h, w = spec["grid"]
    if f * h * w != tokens or 2 * sum(spec["pairs"]) != head_dim:
        raise ValueError("oracle: 3-D grid does not match the tensor")
    return rope_angles_3d(spec["grid"], spec["pairs"], spec["theta"])


def rope_apply(x, angle, inverse=False):
    """D6 on a contiguous [B, T, H, D] tensor -> float64 array of the same shape."""
    X = _In(x)
    if X.t.dim() != 4:
        raise ValueError("oracle: rope expects [batch, tokens, heads, head_dim]")
    b, t, h, d = X.t.shape
    ang = np.ascontiguousarray(angle, dtype=np.float64)
    if ang.shape != (t, d // 2):
        raise ValueError("oracle: angle table shape mismatch")
    out = _out(b, t, h, d)
    lib().oracle_rope_apply(X.p, X.dt, b, t, h, d, _ptr(ang), int(bool(inverse)), _ptr(out))
    return out


def _token_angles(angle, rows, rows_per_token):
    ang = np.ascontiguousarray(angle, dtype=np.float64)
    return ang[np.arange(rows) // rows_per_token]


def rmsnorm_rope_fwd(x, w, angle, head_dim, rows_per_token=1, eps=1e-6, gemma=False):
    """D1 then D6 on its output, in fp64 with no rounding in between.

    x: [rows, n], n a multiple of head_dim; row i uses the angle row
    i // rows_per_token.  Returns (out [rows, n], inv_rms [rows])."""
    y, r = rmsnorm_fwd(x, w, eps, gemma)
    rows, n = y.shape
    ang = _token_angles(angle, rows, rows_per_token)
    out = rope_apply(torch.from_numpy(y).view(1, rows, n // head_dim, head_dim), ang)
    return out.reshape(rows, n), r


def rmsnorm_rope_bwd(dout, x, w, angle, head_dim, rows_per_token=1, eps=1e-6, gemma=False,
                     want_dx=True, want_dw=True):
    """Backward of rmsnorm_rope_fwd: D6 inverse on dout, then D2.  Returns (dx, dw)."""
    rows, n = x.shape
    ang = _token_angles(angle, rows, rows_per_token)
    dy = rope_apply(dout.reshape(1, rows, n // head_dim, head_dim), ang, inverse=True)
    xd = x.detach().cpu().double() if isinstance(x, torch.Tensor) else torch.from_numpy(x)
    return rmsnorm_bwd(torch.from_numpy(dy.reshape(rows, n)), xd, w, eps, gemma,
                       want_dx=want_dx, want_dw=want_dw)


def widen(t) -> np.ndarray:
    """The oracle's exact widening of stored values to float64."""
    T = _In(t)
    out = _out(T.t.numel())
    lib().oracle_widen(T.p, T.dt, T.t.numel(), _ptr(out))
    return out.reshape(tuple(T.t.shape))


def max_threads() -> int:
    """OpenMP threads the oracle's row loops run on."""
    return int(lib().oracle_max_threads())


def gelu_tanh(v):
    """D7 activation on a scalar (float64)."""
    return lib().oracle_gelu_tanh(float(v))


def gelu_tanh_grad(v):
    """Derivative of D7's activation on a scalar (float64)."""
    return lib().oracle_gelu_tanh_grad(float(v))


def layernorm_gelu_fwd(x, gamma=None, beta=None, eps=1e-5):
    """D7 forward: gelu_tanh(D3(x)) -> (y, mean, rstd) in float64."""
    X, G, B = _In(x), _In(gamma), _In(beta)
    m, n = _rows_n(X.t)
    y, mu, r = _out(m, n), _out(m), _out(m)
    lib().oracle_layernorm_gelu_fwd(X.p, X.dt, G.p, B.p, G.dt if G.t is not None else B.dt,
                                    m, n, float(eps), _ptr(y), _ptr(mu), _ptr(r))
    return y, mu, r


def layernorm_gelu_bwd(dout, x, gamma=None, beta=None, eps=1e-5, want_dx=True, want_dw=True):
    """D7 backward -> (dx, dgamma, dbeta) in float64."""
    DY, X, G, B = _In(dout), _In(x), _In(gamma), _In(beta)
    if DY.dt != X.dt:
        raise TypeError("oracle: dout and x must share a dtype")
    m, n = _rows_n(X.t)
    dx = _out(m, n) if want_dx else None
    dg = _out(n) if want_dw else None
    db = _out(n) if want_dw else None
    lib().oracle_layernorm_gelu_bwd(DY.p, X.p, X.dt, G.p, B.p, G.dt if G.t is not None else B.dt,
                                    m, n, float(eps), _ptr(dx), _ptr(dg), _ptr(db))
    return dx, dg, db


def rmsnorm_linear(x, w, W, eps=1e-6, gemma=False):
    """D1 followed by the linear layer y @ W^T, in float64 with no rounding in
    between; W is [N, K].  Returns (out [rows, N], inv_rms [rows], S) where
    S = |y| @ |W|^T bounds each output's rounding sensitivity (the sum of
    the magnitudes of its K products)."""
    y, r = rmsnorm_fwd(x, w, eps, gemma)
    Wd = W.detach().cpu().double().numpy() if isinstance(W, torch.Tensor) else np.asarray(W, np.float64)
    return y @ Wd.T, r, np.abs(y) @ np.abs(Wd).T


def layernorm_linear(x, gamma, beta, W, eps=1e-5):
    """D3 followed by the linear layer y @ W^T, in float64 with no rounding in
    between (the LayerNorm fused with the linear layer after it,
    "HY-Motion 1.0性能优化", 3.1 算子融合与计算图优化); W is [N, K].  Returns
    (out [rows, N], mean [rows], rstd [rows])."""
    y, mu, rs = layernorm_fwd(x, gamma, beta, eps)
    Wd = W.detach().cpu().double().numpy() if isinstance(W, torch.Tensor) else np.asarray(W, np.float64)
    return y @ Wd.T, mu, rs
