"""Parity bounds used by the GPU tests (kept in one place, written out here).

R is the oracle's float64 value (never rounded to the storage type), O the
GPU output widened exactly to float64, s a scale for the row the element
belongs to (the RMS of R over that row; for RoPE the row is one head vector;
for a column-gradient vector, the RMS of the whole vector).

  fp32 outputs              |O - R| <= 1e-5 (|R| + s)
  column gradients (fp32)   |O - R| <= 1e-4 (|R| + s)
  bf16 outputs              |O - R| <= ulp_bf16(R) + 1e-5 s      ("1 bf16 ulp")
  fp16 outputs              |O - R| <= ulp_f16(R) + 1e-5 s       ("1 fp16 ulp")

  per-row statistics        |O - R| <= 1e-5 (|R| + s), s = 0 except for the
                            LayerNorm mean, whose s is the RMS of the x row

For an input gradient dx the row scale s is the RMS of r * dy * w' over the
row (the terms dx is the difference of) rather than the RMS of dx itself:
dx can cancel far below its terms, and fp32 arithmetic is accurate relative
to the terms only.  On ordinary rows the two scales are of the same size.

ulp_bf16(R) = 2^(floor(log2 |R|) - 7): bf16 keeps 8 significant bits, so this
is the spacing of bf16 numbers in R's binade (2^-7 ~ 7.8e-3 relative at its
bottom).  Rounding a value computed in fp32 once, to nearest, stays within
half of it plus the fp32 error, so one ulp leaves room only for that.
"""
import numpy as np
import torch


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().to("cpu", torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def ulp_bf16(r: np.ndarray) -> np.ndarray:
    a = np.abs(r)
    _, e = np.frexp(a)              # a = m 2^e, m in [0.5, 1): floor(log2 a) = e - 1
    u = np.ldexp(1.0, e - 8)
    return np.where(a > 0, u, 0.0)


def ulp_f16(r: np.ndarray) -> np.ndarray:
    """Spacing of IEEE binary16 numbers at R: 11 significant bits, so
    2^(floor(log2 |R|) - 10) for normal values and 2^-24 below 2^-14."""
    a = np.abs(r)
    _, e = np.frexp(a)
    return np.ldexp(1.0, np.maximum(e - 11, -24))


def row_rms(r: np.ndarray) -> np.ndarray:
    """RMS over the last axis, broadcastable against r."""
    return np.sqrt(np.mean(r * r, axis=-1, keepdims=True))


def _report(name, o, r, err, tol):
    bad = err > tol
    i = np.unravel_index(np.argmax(err - tol), err.shape)
    return (f"{name}: {int(bad.sum())} of {err.size} outside the bound; worst at {i}: "
            f"gpu={o[i]!r} oracle={r[i]!r} err={err[i]:.3e} bound={tol[i]:.3e}")


def check(name, o, r, kind, s=None, extra=None):
    """Assert the bound of `kind` ('f32', 'bf16', 'col', 'stat') element-wise.

    extra: an additional absolute allowance derived for chained checks."""
    o, r = to64(o), to64(r)
    assert o.shape == r.shape, f"{name}: shape {o.shape} vs {r.shape}"
    if s is None:
        s = row_rms(r) if kind in ("f32", "bf16", "f16") else np.sqrt(np.mean(r * r))
    err = np.abs(o - r)
    if kind == "bf16":
        tol = ulp_bf16(r) + 1e-5 * s
    elif kind == "f16":
        tol = ulp_f16(r) + 1e-5 * s
    elif kind == "col":
        tol = 1e-4 * (np.abs(r) + s)
    else:  # f32, stat
        tol = 1e-5 * (np.abs(r) + s)
    if extra is not None:
        tol = tol + extra
    tol = np.broadcast_to(tol, err.shape)
    assert np.all(np.isfinite(o)), f"{name}: non-finite GPU output"
    assert np.all(err <= tol), _report(name, o, r, err, tol)
    return float(np.max(err / np.maximum(tol, 1e-300)))


def out_kind(dtype) -> str:
    return {torch.bfloat16: "bf16", torch.float16: "f16"}.get(dtype, "f32")


def grad_scale(r, dy, w, gemma=False):
    """Row scale for dx: RMS over the row of r * dy * w' (the terms dx is a
    difference of).  dx can cancel to far below this (a one-column row, where
    RMSNorm's dx is ~eps-sized and LayerNorm's is exactly 0), and fp32 is only
    accurate relative to the terms, so the bound is scaled by them."""
    wp = np.ones(dy.shape[-1]) if w is None else to64(w) + (1.0 if gemma else 0.0)
    t = to64(r)[:, None] * to64(dy).reshape(len(r), -1) * wp[None, :]
    return np.sqrt(np.mean(t * t, axis=1, keepdims=True))
