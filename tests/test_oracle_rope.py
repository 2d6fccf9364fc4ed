"""Pins for the fp64 RoPE oracle (CPU only).

The rotation is checked against complex multiplication done by PyTorch in
complex128 (which fixes the interleaved real/imaginary convention and the
sign), the pair-norm and inverse invariants, the quarter-turn special case,
composition of angles, the Jacobian-transpose property of the inverse, and a
hand-derived worked example.  The angle tables are checked against their
structure: zero at position 0, linear in position, geometric across pairs,
and each 3-D axis block equal to a 1-D table of that axis.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _x(shape, seed):
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape))


def _cases(op):
    with open(GOLD) as f:
        return [c for c in json.load(f)["cases"] if c["op"] == op]


def test_golden_rope():
    for op, inv in (("rope_fwd_1d", False), ("rope_inverse_1d", True)):
        for c in _cases(op):
            d = c["head_dim"]
            ang = oracle.rope_angles_1d(c["position"] + 1, d, 0, c["theta"])[c["position"]:]
            x = torch.tensor(c["x"], dtype=torch.float64).view(1, 1, 1, d)
            out = oracle.rope_apply(x, ang, inverse=inv)
            np.testing.assert_allclose(out.reshape(-1), c["out"], rtol=1e-14, atol=1e-16)


def test_angles_1d_structure():
    d, t, theta = 128, 50, 10000.0
    a = oracle.rope_angles_1d(t, d, 0, theta)
    assert a.shape == (t, d // 2)
    assert np.all(a[0] == 0.0)                       # position 0: no rotation
    np.testing.assert_allclose(a[:, 0], np.arange(t), rtol=0, atol=0)   # first pair: unit frequency
    np.testing.assert_allclose(a, np.arange(t)[:, None] * a[1][None, :], rtol=1e-15)  # linear in pos
    ratio = a[1, 1:] / a[1, :-1]                      # geometric across pairs
    np.testing.assert_allclose(ratio, ratio[0], rtol=1e-13)
    assert abs(a[1, d // 4] - 1.0 / math.sqrt(theta)) < 1e-16   # middle pair: theta^(-1/2) = 0.01
    b = oracle.rope_angles_1d(10, d, 40, theta)       # pos0 offsets the positions
    np.testing.assert_array_equal(b, a[40:50] if t > 50 else oracle.rope_angles_1d(50, d, 0, theta)[40:50])


def test_angles_3d_axis_blocks():
    grid, pairs, theta = (3, 4, 5), (5, 4, 3), 10000.0
    a = oracle.rope_angles_3d(grid, pairs, theta)
    f_, h_, w_ = grid
    pt, ph, pw = pairs
    a = a.reshape(f_, h_, w_, pt + ph + pw)
    t1 = oracle.rope_angles_1d(f_, 2 * pt, 0, theta)
    h1 = oracle.rope_angles_1d(h_, 2 * ph, 0, theta)
    w1 = oracle.rope_angles_1d(w_, 2 * pw, 0, theta)
    for f in range(f_):
        for h in range(h_):
            for w in range(w_):
                np.testing.assert_allclose(a[f, h, w, :pt], t1[f], rtol=1e-15)
                np.testing.assert_allclose(a[f, h, w, pt:pt + ph], h1[h], rtol=1e-15)
                np.testing.assert_allclose(a[f, h, w, pt + ph:], w1[w], rtol=1e-15)
    assert np.all(a[0, 0, 0] == 0.0)


def test_apply_vs_complex_multiplication():
    b, t, h, d = 2, 7, 3, 16
    x = _x((b, t, h, d), 1)
    ang = oracle.rope_angles_1d(t, d, 3, 10000.0)
    phi = torch.from_numpy(ang)[None, :, None, :]
    z = torch.view_as_complex(x.view(b, t, h, d // 2, 2).contiguous())
    for inv in (False, True):
        rot = torch.polar(torch.ones_like(phi), -phi if inv else phi)
        ref = torch.view_as_real(z * rot).reshape(b, t, h, d)
        np.testing.assert_allclose(oracle.rope_apply(x, ang, inv), ref.numpy(), rtol=1e-13, atol=1e-14)


def test_apply_invariants():
    b, t, h, d = 1, 9, 2, 12
    x = _x((b, t, h, d), 2)
    ang = oracle.rope_angles_1d(t, d, 0, 500.0)
    y = oracle.rope_apply(x, ang)
    pn = lambda v: (v.reshape(-1, 2) ** 2).sum(axis=1)
    np.testing.assert_allclose(pn(y), pn(x.numpy()), rtol=1e-13)             # pair norms kept
    back = oracle.rope_apply(torch.from_numpy(y), ang, inverse=True)
    np.testing.assert_allclose(back, x.numpy(), rtol=1e-13, atol=1e-14)       # inverse recovers x
    np.testing.assert_array_equal(y[:, 0], x.numpy()[:, 0])                   # position 0 identity


def test_quarter_turn_and_composition():
    d = 6
    x = _x((1, 1, 4, d), 3)
    quarter = np.full((1, d // 2), math.pi / 2)
    y = oracle.rope_apply(x, quarter).reshape(-1, 2)
    xv = x.numpy().reshape(-1, 2)
    np.testing.assert_allclose(y, np.stack([-xv[:, 1], xv[:, 0]], axis=1), atol=1e-15)
    p1, p2 = np.array([[0.3, -1.1, 2.5]]), np.array([[0.9, 0.4, -3.0]])
    two = oracle.rope_apply(torch.from_numpy(oracle.rope_apply(x, p1)), p2)
    one = oracle.rope_apply(x, p1 + p2)
    np.testing.assert_allclose(two, one, rtol=1e-13, atol=1e-14)


def test_inverse_is_jacobian_transpose():
    # forward is linear in x; the backward of a linear map is its transpose,
    # and the pages use the inverse as the backward
    d, h = 8, 2
    ang = oracle.rope_angles_1d(3, d, 0, 10000.0)[2:3]
    n = h * d

    def mat(inv):
        cols = []
        for k in range(n):
            e = torch.zeros(n, dtype=torch.float64)
            e[k] = 1.0
            cols.append(oracle.rope_apply(e.view(1, 1, h, d), ang, inv).reshape(-1))
        return np.stack(cols, axis=1)

    np.testing.assert_allclose(mat(True), mat(False).T, atol=1e-15)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_apply_reads_storage_dtype_exactly(dtype):
    x = _x((1, 4, 2, 8), 4).to(dtype)
    ang = oracle.rope_angles_1d(4, 8, 0, 10000.0)
    np.testing.assert_array_equal(oracle.rope_apply(x, ang), oracle.rope_apply(x.double(), ang))
