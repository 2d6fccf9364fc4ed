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
    """2^(floor(log2 |R|) - 7), 0 for R = 0: the float64 exponent field alone
    (sign and significand masked off) is 2^floor(log2 |R|) for normal R."""
    a = np.ascontiguousarray(r, dtype=np.float64)
    p2 = (a.view(np.int64) & np.int64(0x7FF0000000000000)).view(np.float64)
    return p2 * 2.0 ** -7


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


# Constants of the bound for a norm folded into a linear layer (below).
LIN_C1 = 6.0  # rounding of the folded weight: 6 x the scale of K independent roundings
LIN_C2 = 8.0  # fp32 accumulation: probabilistic bound lambda sqrt(K) u S, lambda = 8


def linear_extra(R, y, W, folded):
    """Allowance beyond one bf16 ulp for an output of a norm folded into the
    following linear layer, out[m][n] = sum_k y[m][k] W[n][k] with y the fp64
    normalised row, computed on the matrix cores from bf16 operands.

    With p_k = y_k W[n][k]:
      * the norm weight folded into W is rounded once to bf16, a relative
        error d_k with |d_k| <= 2^-9 per product; the error sum_k p_k d_k of
        K independent roundings stays within LIN_C1 2^-9 sqrt(sum_k p_k^2)
        (Hoeffding: probability <= 2 exp(-LIN_C1^2 / 2) ~ 3e-8 per element;
        as a normal approximation, over 10 standard deviations).  Without a
        norm weight the bf16 W enters exactly and this term is 0;
      * the K products (exact in fp32) are added in fp32 in an order the
        hardware fixes: within LIN_C2 sqrt(K) 2^-24 S, S = sum_k |p_k|
        (probabilistic rounding-error bound with lambda = LIN_C2; the
        worst-case K 2^-24 S would exceed a bf16 ulp at long K);
      * the row statistic multiplies the sum: its relative error is held to
        1e-5 by the statistics check, hence 1e-5 |R|.
    """
    y, Wd = to64(y), to64(W)
    K = Wd.shape[1]
    S = np.abs(y) @ np.abs(Wd).T
    extra = 1e-5 * np.abs(R) + LIN_C2 * np.sqrt(K) * 2.0 ** -24 * S
    if folded:
        extra = extra + LIN_C1 * 2.0 ** -9 * np.sqrt((y * y) @ (Wd * Wd).T)
    return extra


def ln_linear_extra(R, x, mean, rstd, gamma, beta, W):
    """Allowance beyond one bf16 ulp for an output of LayerNorm folded into
    the following linear layer, evaluated on the matrix cores as
    r_m (sum_k x[m][k] Wf[n][k] - mu_m c_n) + d_n with Wf = bf16(gamma W),
    c_n = sum_k Wf[n][k], d_n = sum_k beta_k W[n][k] (fp32 sums).  mean and
    rstd are the oracle's fp64 statistics.  With g = gamma (1 when none):
      * the folded weight's one rounding: LIN_C1 2^-9 sqrt(sum_k p_k^2),
        p_k = (x_k - mu) r g_k W[n][k] (0 without gamma: W enters exactly);
      * the fp32 sums, LIN_C2 sqrt(K) 2^-24 times the magnitude sum of what
        each adds: r sum_k |x_k g_k W[n][k]| (the product, of the uncentred
        x), r |mu| sum_k |g_k W[n][k]| (c_n), sum_k |beta_k W[n][k]| (d_n),
        plus a few fp32 roundings of those terms in the epilogue;
      * the statistics, held to 1e-5 by their own checks: 1e-5 |R - d| from
        r, and 1e-5 rms(x) r |c_n| from the mean.
    """
    x, Wd = to64(x), to64(W)
    K = Wd.shape[1]
    mu, r = to64(mean)[:, None], to64(rstd)[:, None]
    g = np.ones(K) if gamma is None else to64(gamma)
    b = np.zeros(K) if beta is None else to64(beta)
    gW = np.abs(Wd * g[None, :])
    Sx = np.abs(x) @ gW.T
    Sc = gW.sum(axis=1)[None, :]
    Sd = (np.abs(Wd) @ np.abs(b))[None, :]
    d = (Wd @ b)[None, :]
    c = (Wd * g[None, :]).sum(axis=1)[None, :]
    sums = r * Sx + r * np.abs(mu) * Sc + Sd
    extra = (LIN_C2 * np.sqrt(K) + 4.0) * 2.0 ** -24 * sums
    extra = extra + 1e-5 * (np.abs(R) + np.abs(d))
    extra = extra + 1e-5 * np.sqrt(np.mean(x * x, axis=1, keepdims=True)) * r * np.abs(c)
    if gamma is not None:
        xc = (x - mu) * r * g[None, :]
        extra = extra + LIN_C1 * 2.0 ** -9 * np.sqrt((xc * xc) @ (Wd * Wd).T)
    return extra
