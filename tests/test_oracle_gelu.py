"""Pins for the oracle's LayerNorm + tanh-GeLU (CPU only): the activation
against PyTorch's float64 tanh-GeLU and its exact symmetry
gelu(v) - gelu(-v) = v; its derivative against finite differences and
autograd; the fused forward against layer_norm followed by gelu; the
backward against float64 autograd and finite differences."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _x(shape, seed, mean=0.0, std=1.0):
    return torch.from_numpy(mean + std * np.random.default_rng(seed).standard_normal(shape))


def test_activation_against_torch_and_symmetry():
    v = np.concatenate([np.linspace(-8, 8, 161), [0.0, 1e-3, -1e-3, 30.0, -30.0]])
    ours = np.array([oracle.gelu_tanh(t) for t in v])
    ref = F.gelu(torch.from_numpy(v), approximate="tanh").numpy()
    # the printed form 0.5 v (1 + tanh u) cancels for v << 0, so agreement is
    # absolute there: a few double roundings of v
    np.testing.assert_allclose(ours, ref, rtol=1e-14, atol=4e-15)
    for t in v:
        assert abs((oracle.gelu_tanh(t) - oracle.gelu_tanh(-t)) - t) <= 1e-15 * (1 + abs(t))
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh_grad(0.0) == 0.5


def test_activation_derivative():
    v = torch.linspace(-6, 6, 97, dtype=torch.float64, requires_grad=True)
    F.gelu(v, approximate="tanh").sum().backward()
    ours = np.array([oracle.gelu_tanh_grad(t) for t in v.detach().numpy()])
    np.testing.assert_allclose(ours, v.grad.numpy(), rtol=1e-13, atol=1e-15)
    h = 1e-6
    for t in (-3.3, -0.7, 0.0, 0.4, 2.9):
        fd = (oracle.gelu_tanh(t + h) - oracle.gelu_tanh(t - h)) / (2 * h)
        assert abs(fd - oracle.gelu_tanh_grad(t)) < 1e-8


def test_fused_forward():
    x, g, b = _x((7, 48), 1, 0.5, 2.0), _x(48, 2, 1.0, 0.1), _x(48, 3, 0.0, 0.1)
    y, mu, r = oracle.layernorm_gelu_fwd(x, g, b, 1e-5)
    ref = F.gelu(F.layer_norm(x, (48,), g, b, 1e-5), approximate="tanh")
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)
    _, mu2, r2 = oracle.layernorm_fwd(x, g, b, 1e-5)
    assert np.array_equal(mu, mu2) and np.array_equal(r, r2)


def test_fused_backward_autograd():
    x, g, b, d = _x((6, 40), 4, 0.5, 2.0), _x(40, 5, 1.0, 0.1), _x(40, 6, 0.0, 0.3), _x((6, 40), 7)
    xa, ga, ba = (t.clone().requires_grad_() for t in (x, g, b))
    F.gelu(F.layer_norm(xa, (40,), ga, ba, 1e-5), approximate="tanh").backward(d)
    dx, dg, db = oracle.layernorm_gelu_bwd(d, x, g, b, 1e-5)
    np.testing.assert_allclose(dx, xa.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dg, ga.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(db, ba.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_fused_backward_finite_differences():
    x, g, b, d = _x((3, 8), 8, 0.5, 2.0), _x(8, 9, 1.0, 0.3), _x(8, 10, 0.0, 0.3), _x((3, 8), 11)
    dx, dg, db = oracle.layernorm_gelu_bwd(d, x, g, b, 1e-3)

    def loss():
        y, _, _ = oracle.layernorm_gelu_fwd(x, g, b, 1e-3)
        return float((y * d.numpy()).sum())

    h = 1e-6
    for t, grad in ((x, dx), (g, dg), (b, db)):
        flat = t.view(-1)
        for i in range(flat.numel()):
            old = flat[i].item()
            flat[i] = old + h
            fp = loss()
            flat[i] = old - h
            fm = loss()
            flat[i] = old
            assert abs((fp - fm) / (2 * h) - np.asarray(grad).reshape(-1)[i]) < 1e-6 * (1 + abs(np.asarray(grad).reshape(-1)[i]))
