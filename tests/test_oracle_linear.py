"""Pins for the oracle's RMSNorm -> linear composition (CPU only): brute
force on a tiny case, the identity weight reducing it to RMSNorm, and
linearity in W."""
import numpy as np
import torch

import oracle


def _x(shape, seed, scale=1.0):
    return torch.from_numpy(scale * np.random.default_rng(seed).standard_normal(shape))


def test_brute_force_tiny():
    x, w, W = _x((3, 5), 1), _x(5, 2, 0.1) + 1.0, _x((4, 5), 3)
    out, r, S = oracle.rmsnorm_linear(x, w, W, eps=1e-6)
    for m in range(3):
        ms = sum(float(x[m, k]) ** 2 for k in range(5)) / 5
        rm = 1.0 / (ms + 1e-6) ** 0.5
        assert abs(r[m] - rm) <= 1e-15 * rm
        for n in range(4):
            terms = [float(x[m, k]) * rm * float(w[k]) * float(W[n, k]) for k in range(5)]
            assert abs(out[m, n] - sum(terms)) <= 1e-14 * sum(abs(t) for t in terms)
            assert abs(S[m, n] - sum(abs(t) for t in terms)) <= 1e-14 * S[m, n]


def test_identity_weight_is_rmsnorm_and_gemma():
    x, w = _x((6, 16), 4), _x(16, 5, 0.1)
    out, r, _ = oracle.rmsnorm_linear(x, w, torch.eye(16, dtype=torch.float64), 1e-5, gemma=True)
    y, r2 = oracle.rmsnorm_fwd(x, w, 1e-5, gemma=True)
    assert np.array_equal(out, y) and np.array_equal(r, r2)


def test_linear_in_W():
    x, w, W1, W2 = _x((5, 8), 6), _x(8, 7, 0.2) + 1, _x((3, 8), 8), _x((3, 8), 9)
    a, _, _ = oracle.rmsnorm_linear(x, w, W1)
    b, _, _ = oracle.rmsnorm_linear(x, w, W2)
    c, _, _ = oracle.rmsnorm_linear(x, w, 2.0 * W1 - W2)
    np.testing.assert_allclose(c, 2.0 * a - b, rtol=1e-12, atol=1e-12)
