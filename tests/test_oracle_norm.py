"""Pins for the fp64 norm oracle (CPU only).

Each test checks the oracle against something other than itself: a closed
form or invariant of the definition, a hand-derived worked example, finite
differences, exactly rounded brute-force sums, or PyTorch's own float64
rms_norm / layer_norm / autograd.  A dropped term, a wrong divisor, eps in the
wrong place or a sign error in the backward fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _f64(shape, seed, mean=0.0, std=1.0):
    g = np.random.default_rng(seed)
    return torch.from_numpy(mean + std * g.standard_normal(shape))


def _cases(op):
    with open(GOLD) as f:
        return [c for c in json.load(f)["cases"] if c["op"] == op]


# ---------------------------------------------------------------- worked examples

def test_golden_rmsnorm():
    for c in _cases("rmsnorm_fwd"):
        y, r = oracle.rmsnorm_fwd(torch.tensor(c["x"], dtype=torch.float64), eps=c["eps"])
        np.testing.assert_allclose(y, c["y"], rtol=1e-14)
        np.testing.assert_allclose(r, c["inv_rms"], rtol=1e-14)
    for c in _cases("rmsnorm_fwd_gemma"):
        y, _ = oracle.rmsnorm_fwd(torch.tensor(c["x"], dtype=torch.float64),
                                  torch.tensor(c["w"], dtype=torch.float64), eps=c["eps"], gemma=True)
        np.testing.assert_allclose(y, c["y"], rtol=1e-14)


def test_golden_layernorm():
    for c in _cases("layernorm_fwd"):
        y, mu, r = oracle.layernorm_fwd(torch.tensor(c["x"], dtype=torch.float64), eps=c["eps"])
        np.testing.assert_allclose(y, c["y"], rtol=1e-14)
        np.testing.assert_allclose(mu, c["mean"], rtol=1e-15)
        np.testing.assert_allclose(r, c["rstd"], rtol=1e-14)


# ---------------------------------------------------------------- RMSNorm forward

@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_rms_unit_rms_closed_form(eps):
    x = _f64((7, 33), 1)
    y, r = oracle.rmsnorm_fwd(x, eps=eps)
    ms = (x.numpy() ** 2).mean(axis=1)
    # with no weight, mean(y^2) = ms / (ms + eps) exactly in real arithmetic
    np.testing.assert_allclose((y ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-13)
    # y is x scaled by the cached statistic
    np.testing.assert_allclose(y, x.numpy() * r[:, None], rtol=1e-15)


def test_rms_scale_invariance_and_constant_row():
    x = _f64((5, 16), 2)
    y1, _ = oracle.rmsnorm_fwd(x, eps=0.0)
    y2, _ = oracle.rmsnorm_fwd(37.5 * x, eps=0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-13)
    c, eps = 0.3, 1e-2
    w = _f64(16, 3)
    y, _ = oracle.rmsnorm_fwd(torch.full((2, 16), c, dtype=torch.float64), w, eps=eps)
    np.testing.assert_allclose(y, np.broadcast_to(c / math.sqrt(c * c + eps) * w.numpy(), (2, 16)),
                               rtol=1e-14)


def test_rms_gemma_offset():
    x = _f64((4, 24), 4)
    zero = torch.zeros(24, dtype=torch.float64)
    one = torch.ones(24, dtype=torch.float64)
    a, _ = oracle.rmsnorm_fwd(x, zero, eps=1e-6, gemma=True)
    b, _ = oracle.rmsnorm_fwd(x, one, eps=1e-6, gemma=False)
    assert np.array_equal(a, b)
    w = _f64(24, 5)
    c, _ = oracle.rmsnorm_fwd(x, w, eps=1e-6, gemma=True)
    d, _ = oracle.rmsnorm_fwd(x, 1.0 + w, eps=1e-6, gemma=False)
    np.testing.assert_allclose(c, d, rtol=1e-15, atol=1e-15)


@pytest.mark.parametrize("gemma", [False, True])
def test_rms_fwd_vs_torch(gemma):
    x, w = _f64((9, 40), 6), _f64(40, 7, 1.0, 0.1)
    y, _ = oracle.rmsnorm_fwd(x, w, eps=1e-6, gemma=gemma)
    ref = F.rms_norm(x, (40,), weight=(1.0 + w) if gemma else w, eps=1e-6)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- RMSNorm backward

def _fd_grad(fun, t, h=1e-6):
    g = torch.zeros_like(t)
    flat, gf = t.view(-1), g.view(-1)
    for i in range(flat.numel()):
        old = flat[i].item()
        flat[i] = old + h
        fp = fun()
        flat[i] = old - h
        fm = fun()
        flat[i] = old
        gf[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("gemma", [False, True])
def test_rms_bwd_finite_differences(gemma):
    x, w, dy = _f64((3, 8), 8), _f64(8, 9, 1.0, 0.3), _f64((3, 8), 10)
    eps = 1e-3
    dx, dw = oracle.rmsnorm_bwd(dy, x, w, eps=eps, gemma=gemma)

    def loss():
        y, _ = oracle.rmsnorm_fwd(x, w, eps=eps, gemma=gemma)
        return float((y * dy.numpy()).sum())

    np.testing.assert_allclose(dx, _fd_grad(loss, x).numpy(), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, _fd_grad(loss, w).numpy(), rtol=1e-6, atol=1e-8)


@pytest.mark.parametrize("eps", [0.0, 1e-2])
def test_rms_bwd_radial_invariant(eps):
    # along the row itself y only changes through eps, so
    # sum_j x dx = eps r^2 sum_j g xhat (and 0 when eps = 0)
    x, w, dy = _f64((6, 20), 11), _f64(20, 12), _f64((6, 20), 13)
    dx, _ = oracle.rmsnorm_bwd(dy, x, w, eps=eps)
    _, r = oracle.rmsnorm_fwd(x, eps=eps)
    g = dy.numpy() * w.numpy()
    xhat = x.numpy() * r[:, None]
    lhs = (x.numpy() * dx).sum(axis=1)
    rhs = eps * r ** 2 * (g * xhat).sum(axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("gemma", [False, True])
def test_rms_bwd_vs_autograd(gemma):
    x, w, dy = _f64((5, 48), 14), _f64(48, 15, 0.0, 0.2), _f64((5, 48), 16)
    xa, wa = x.clone().requires_grad_(), w.clone().requires_grad_()
    F.rms_norm(xa, (48,), weight=(1.0 + wa) if gemma else wa, eps=1e-6).backward(dy)
    dx, dw = oracle.rmsnorm_bwd(dy, x, w, eps=1e-6, gemma=gemma)
    np.testing.assert_allclose(dx, xa.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw, wa.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_rms_dw_exact_column_sums_bf16():
    # dw against exactly rounded (math.fsum) column sums of the products
    from workloads import norm_inputs
    inp = norm_inputs("tiny_f32")
    x, dy = inp["x"][:32, :48].to(torch.bfloat16), inp["dy"][:32, :48].to(torch.bfloat16)
    _, dw = oracle.rmsnorm_bwd(dy, x, None, eps=1e-6)
    _, r = oracle.rmsnorm_fwd(x, eps=1e-6)
    xd, dyd = x.double().numpy(), dy.double().numpy()
    for j in range(48):
        ref = math.fsum(dyd[i, j] * (xd[i, j] * r[i]) for i in range(32))
        assert abs(dw[j] - ref) <= 1e-13 * (abs(ref) + 1.0)


def test_rms_non_affine_bwd():
    x, dy = _f64((4, 12), 17), _f64((4, 12), 18)
    dx1, dw = oracle.rmsnorm_bwd(dy, x, None, eps=1e-6, want_dw=False)
    dx2, _ = oracle.rmsnorm_bwd(dy, x, torch.ones(12, dtype=torch.float64), eps=1e-6)
    assert dw is None
    assert np.array_equal(dx1, dx2)


# ---------------------------------------------------------------- LayerNorm forward

@pytest.mark.parametrize("eps", [0.0, 1e-5, 0.25])
def test_ln_zero_mean_unit_variance(eps):
    x = _f64((6, 50), 20, 0.5, 2.0)
    y, mu, r = oracle.layernorm_fwd(x, eps=eps)
    var = x.numpy().var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
    np.testing.assert_allclose((y ** 2).mean(axis=1), var / (var + eps), rtol=1e-13)
    np.testing.assert_allclose(mu, x.numpy().mean(axis=1), rtol=1e-14, atol=1e-14)


def test_ln_constant_row_and_single_column():
    g, b = _f64(10, 21), _f64(10, 22)
    y, _, _ = oracle.layernorm_fwd(torch.full((3, 10), -1.7, dtype=torch.float64), g, b, eps=1e-5)
    np.testing.assert_allclose(y, np.broadcast_to(b.numpy(), (3, 10)), rtol=0, atol=1e-12)
    y1, _, _ = oracle.layernorm_fwd(_f64((4, 1), 23), g[:1], b[:1], eps=1e-5)
    np.testing.assert_allclose(y1[:, 0], b[0].item(), rtol=0, atol=0)


def test_ln_fwd_vs_torch():
    x, g, b = _f64((8, 64), 24, 0.5, 2.0), _f64(64, 25, 1.0, 0.1), _f64(64, 26, 0.0, 0.1)
    y, mu, r = oracle.layernorm_fwd(x, g, b, eps=1e-5)
    ref = F.layer_norm(x, (64,), g, b, eps=1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)
    v, m = torch.var_mean(x, dim=1, unbiased=False)
    np.testing.assert_allclose(mu, m.numpy(), rtol=1e-14)
    np.testing.assert_allclose(r, (1.0 / torch.sqrt(v + 1e-5)).numpy(), rtol=1e-13)


# ---------------------------------------------------------------- LayerNorm backward

def test_ln_bwd_invariants():
    x, g, dy = _f64((5, 30), 27, 0.5, 2.0), _f64(30, 28), _f64((5, 30), 29)
    eps = 1e-2
    dx, dg, db = oracle.layernorm_bwd(dy, x, g, eps=eps)
    # shift invariance: sum_j dx = 0 exactly in real arithmetic, with any eps
    np.testing.assert_allclose(dx.sum(axis=1), 0.0, atol=1e-12)
    # radial direction: sum_j (x - mu) dx = eps r^2 sum_j g xhat
    _, mu, r = oracle.layernorm_fwd(x, eps=eps)
    xc = x.numpy() - mu[:, None]
    gg = dy.numpy() * g.numpy()
    lhs = (xc * dx).sum(axis=1)
    rhs = eps * r ** 2 * (gg * xc * r[:, None]).sum(axis=1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9, atol=1e-12)
    # dbeta is the column sum of dy (exactly rounded reference)
    dyn = dy.numpy()
    for j in range(30):
        assert abs(db[j] - math.fsum(dyn[:, j])) <= 1e-14 * (1 + abs(db[j]))


def test_ln_bwd_finite_differences():
    x, g, b, dy = _f64((3, 8), 30, 0.5, 2.0), _f64(8, 31, 1.0, 0.3), _f64(8, 32), _f64((3, 8), 33)
    eps = 1e-3
    dx, dg, db = oracle.layernorm_bwd(dy, x, g, eps=eps)

    def loss():
        y, _, _ = oracle.layernorm_fwd(x, g, b, eps=eps)
        return float((y * dy.numpy()).sum())

    np.testing.assert_allclose(dx, _fd_grad(loss, x).numpy(), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dg, _fd_grad(loss, g).numpy(), rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(db, _fd_grad(loss, b).numpy(), rtol=1e-6, atol=1e-8)


def test_ln_bwd_vs_autograd():
    x, g, b, dy = (_f64((6, 40), 34, 0.5, 2.0), _f64(40, 35, 1.0, 0.1), _f64(40, 36),
                   _f64((6, 40), 37))
    xa, ga, ba = (t.clone().requires_grad_() for t in (x, g, b))
    F.layer_norm(xa, (40,), ga, ba, eps=1e-5).backward(dy)
    dx, dg, db = oracle.layernorm_bwd(dy, x, g, eps=1e-5)
    np.testing.assert_allclose(dx, xa.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dg, ga.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, ba.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_inputs_widened_exactly():
    # bf16 and fp32 inputs must reach the oracle bit-exactly (no re-rounding)
    x = _f64((3, 16), 38).to(torch.bfloat16)
    a, ra = oracle.rmsnorm_fwd(x, eps=1e-6)
    b, rb = oracle.rmsnorm_fwd(x.double(), eps=1e-6)
    assert np.array_equal(a, b) and np.array_equal(ra, rb)
    xf = _f64((3, 16), 39).float()
    a, _, _ = oracle.layernorm_fwd(xf, eps=1e-5)
    b, _, _ = oracle.layernorm_fwd(xf.double(), eps=1e-5)
    assert np.array_equal(a, b)


def test_half_inputs_widened_exactly():
    # every one of the 65536 binary16 bit patterns widens to the value
    # torch's own (exact) float16 -> float64 conversion gives: normals,
    # subnormals, signed zeros, infinities; NaN patterns stay NaN
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    h = bits.view(torch.float16)
    got = oracle.widen(h)
    want = h.double().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # and through an operator: fp16 input == its fp64 widening
    x = _f64((3, 16), 40).to(torch.float16)
    a, _, _ = oracle.layernorm_fwd(x, eps=1e-5)
    b, _, _ = oracle.layernorm_fwd(x.double(), eps=1e-5)
    assert np.array_equal(a, b)
    # bf16 through the same entry point
    xb = _f64((2, 8), 41).to(torch.bfloat16)
    assert np.array_equal(oracle.widen(xb), xb.double().numpy())
