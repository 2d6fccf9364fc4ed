"""Pins for the oracle's fused RMSNorm + RoPE (the composition of D1 and D6,
and of D6 inverse and D2), CPU only: zero angles reduce it to RMSNorm, finite
differences give its backward, and PyTorch float64 autograd through
rms_norm and a complex128 rotation agrees with both directions."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _x(shape, seed, scale=1.0):
    return torch.from_numpy(scale * np.random.default_rng(seed).standard_normal(shape))


def test_zero_angles_is_rmsnorm():
    x, w = _x((6, 24), 1), _x(24, 2, 0.1) + 1.0
    ang = np.zeros((6, 4))
    y, r = oracle.rmsnorm_rope_fwd(x, w, ang, head_dim=8)
    y0, r0 = oracle.rmsnorm_fwd(x, w, 1e-6)
    assert np.array_equal(y, y0) and np.array_equal(r, r0)


@pytest.mark.parametrize("rows_per_token", [1, 3])
def test_fused_vs_autograd(rows_per_token):
    rows, d = 6, 8
    n = d * (3 if rows_per_token == 1 else 1)
    x, w, dout = _x((rows, n), 3), _x(n, 4, 0.2) + 1.0, _x((rows, n), 5)
    ang = oracle.rope_angles_1d(rows // rows_per_token, d, 7, 500.0)
    y, _ = oracle.rmsnorm_rope_fwd(x, w, ang, d, rows_per_token)
    dx, dw = oracle.rmsnorm_rope_bwd(dout, x, w, ang, d, rows_per_token)
    xa, wa = x.clone().requires_grad_(), w.clone().requires_grad_()
    yn = F.rms_norm(xa, (n,), weight=wa, eps=1e-6)
    phi = torch.from_numpy(ang[np.arange(rows) // rows_per_token])[:, None, :]
    z = torch.view_as_complex(yn.view(rows, n // d, d // 2, 2)) * torch.polar(torch.ones_like(phi), phi)
    ref = torch.view_as_real(z).reshape(rows, n)
    np.testing.assert_allclose(y, ref.detach().numpy(), rtol=1e-12, atol=1e-13)
    ref.backward(dout)
    np.testing.assert_allclose(dx, xa.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dw, wa.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_fused_bwd_finite_differences():
    rows, d, n = 3, 4, 8
    x, w, dout = _x((rows, n), 6), _x(n, 7, 0.3) + 1.0, _x((rows, n), 8)
    ang = oracle.rope_angles_1d(rows, d, 2, 100.0)
    dx, dw = oracle.rmsnorm_rope_bwd(dout, x, w, ang, d, eps=1e-3, gemma=False)

    def loss():
        y, _ = oracle.rmsnorm_rope_fwd(x, w, ang, d, eps=1e-3)
        return float((y * dout.numpy()).sum())

    h = 1e-6
    for t, g in ((x, dx), (w, dw)):
        flat = t.view(-1)
        fd = np.zeros(flat.numel())
        for i in range(flat.numel()):
            old = flat[i].item()
            flat[i] = old + h
            fp = loss()
            flat[i] = old - h
            fm = loss()
            flat[i] = old
            fd[i] = (fp - fm) / (2 * h)
        np.testing.assert_allclose(np.asarray(g).reshape(-1), fd, rtol=1e-6, atol=1e-8)
