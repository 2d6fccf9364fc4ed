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


# ---- the GPU test's bound for the fused norm -> linear output bites --------
#
# tolerance.linear_extra bounds the fused output against this composition.
# An emulation of the kernel's arithmetic (fold rounded once to bf16, fp32
# sums) must pass it, and plausible kernel mistakes must not: a 16-wide K
# sub-step dropped, the norm weight applied twice, the folded weight rounded
# to a 4-bit significand instead of bf16's 8.  Each output is rounded to
# bf16 as the kernel's is.

import pytest  # noqa: E402

from tolerance import check, linear_extra  # noqa: E402


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def _round_sig(a, bits):
    """Round to nearest with `bits` significant bits (ties away; test aid)."""
    m, e = np.frexp(a)
    return np.ldexp(np.round(m * 2.0 ** bits) / 2.0 ** bits, e)


@pytest.fixture(scope="module")
def case():
    m, n, k = 48, 96, 1024
    rng = np.random.default_rng(4711)
    x = torch.from_numpy(rng.standard_normal((m, k)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(k)).astype(np.float32)).to(torch.bfloat16)
    W = torch.from_numpy((rng.standard_normal((n, k)) / np.sqrt(k)).astype(np.float32)).to(torch.bfloat16)
    R, r, _ = oracle.rmsnorm_linear(x, w, W, 1e-6)
    y, _ = oracle.rmsnorm_fwd(x, w, 1e-6)
    extra = linear_extra(R, y, W, folded=True)
    xd, wd, Wd = (t.double().numpy() for t in (x, w, W))
    return dict(R=R, r=r, y=y, extra=extra, x=xd, w=wd, W=Wd, k=k)


def _kernel_like(c, Wf):
    # bf16 x times the folded weight, products summed in fp32, times r
    acc = (c["x"].astype(np.float32) @ Wf.astype(np.float32).T).astype(np.float64)
    return _bf16(c["r"][:, None] * acc)


def test_bound_admits_the_kernels_arithmetic(case):
    Wf = _bf16(case["W"] * case["w"][None, :])
    check("emulated fused output", _kernel_like(case, Wf), case["R"], "bf16", s=0.0,
          extra=case["extra"])


def test_bound_rejects_a_dropped_k_substep(case):
    c = case
    k0 = 16 * 17
    drop = c["y"][:, k0:k0 + 16] @ c["W"][:, k0:k0 + 16].T
    with pytest.raises(AssertionError, match="outside the bound"):
        check("dropped K step", _bf16(c["R"] - drop), c["R"], "bf16", s=0.0, extra=c["extra"])


def test_bound_rejects_a_twice_applied_norm_weight(case):
    c = case
    Wf = _bf16(_bf16(c["W"] * c["w"][None, :]) * c["w"][None, :])
    with pytest.raises(AssertionError, match="outside the bound"):
        check("norm weight twice", _kernel_like(c, Wf), c["R"], "bf16", s=0.0, extra=c["extra"])


def test_bound_rejects_a_coarser_folded_weight(case):
    c = case
    Wf = _round_sig(c["W"] * c["w"][None, :], 4)
    with pytest.raises(AssertionError, match="outside the bound"):
        check("4-bit folded weight", _kernel_like(c, Wf), c["R"], "bf16", s=0.0, extra=c["extra"])


def test_bound_is_far_tighter_than_the_magnitude_sum(case):
    # the allowance beyond one ulp is about 15% of the worst-case 2^-8 S at
    # K = 1024 (it shrinks as 1/sqrt(K)), about 3 bf16 ulps of a typical output
    S = np.abs(case["y"]) @ np.abs(case["W"]).T
    assert np.median(case["extra"] / (2.0 ** -8 * S)) < 0.2
    assert np.median(case["extra"] / np.abs(case["R"])) < 0.025


# ---- LayerNorm -> linear composition -----------------------------------------

def test_ln_linear_brute_force_tiny():
    x, g, b, W = _x((3, 6), 21, 2.0) + 0.5, _x(6, 22, 0.1) + 1.0, _x(6, 23, 0.1), _x((4, 6), 24)
    out, mu, rs = oracle.layernorm_linear(x, g, b, W, eps=1e-5)
    for m in range(3):
        row = [float(v) for v in x[m]]
        mean = sum(row) / 6
        var = sum((v - mean) ** 2 for v in row) / 6
        r = 1.0 / (var + 1e-5) ** 0.5
        assert abs(mu[m] - mean) <= 1e-15 * (abs(mean) + 1) and abs(rs[m] - r) <= 1e-14 * r
        for n in range(4):
            terms = [((row[k] - mean) * r * float(g[k]) + float(b[k])) * float(W[n, k]) for k in range(6)]
            assert abs(out[m, n] - sum(terms)) <= 1e-13 * sum(abs(t) for t in terms)


def test_ln_linear_identity_weight_is_layernorm():
    x, g, b = _x((5, 16), 25), _x(16, 26, 0.1) + 1, _x(16, 27, 0.1)
    out, mu, rs = oracle.layernorm_linear(x, g, b, torch.eye(16, dtype=torch.float64), 1e-5)
    y, mu2, rs2 = oracle.layernorm_fwd(x, g, b, 1e-5)
    assert np.array_equal(out, y) and np.array_equal(mu, mu2) and np.array_equal(rs, rs2)


def test_ln_linear_is_linear_in_W_and_shift_invariant():
    x, g, b = _x((6, 8), 28), _x(8, 29, 0.2) + 1, _x(8, 30, 0.1)
    W1, W2 = _x((3, 8), 31), _x((3, 8), 32)
    a, _, _ = oracle.layernorm_linear(x, g, b, W1)
    c2, _, _ = oracle.layernorm_linear(x, g, b, W2)
    c, _, _ = oracle.layernorm_linear(x, g, b, 3.0 * W1 - W2)
    np.testing.assert_allclose(c, 3.0 * a - c2, rtol=1e-12, atol=1e-12)
    # a constant added to every element of a row leaves the normalised row,
    # so the output, unchanged
    s, _, _ = oracle.layernorm_linear(x + 7.25, g, b, W1)
    np.testing.assert_allclose(s, a, rtol=1e-9, atol=1e-9)


def test_ln_linear_constant_rows_give_the_bias_through_W():
    x = torch.full((3, 16), 0.75, dtype=torch.float64)
    g, b, W = _x(16, 33, 0.1) + 1, _x(16, 34, 0.1), _x((5, 16), 35)
    out, _, _ = oracle.layernorm_linear(x, g, b, W, 1e-5)
    y, _, _ = oracle.layernorm_fwd(x, g, b, 1e-5)
    assert np.array_equal(y, np.broadcast_to(b.numpy(), y.shape))  # the normalised row is 0
    expect = b.numpy() @ W.numpy().T  # (the matrix product may add in another order)
    np.testing.assert_allclose(out, np.broadcast_to(expect, out.shape), rtol=1e-14, atol=1e-15)
    # no gamma / beta: gamma 1, beta 0 (a constant row then gives exactly 0)
    out0, _, _ = oracle.layernorm_linear(x, None, None, W, 1e-5)
    assert np.array_equal(out0, np.zeros_like(out0))


# ---- the GPU test's bound for the fused LayerNorm -> linear output bites ---

from tolerance import ln_linear_extra  # noqa: E402


@pytest.fixture(scope="module")
def ln_case():
    m, n, k = 48, 96, 1024
    rng = np.random.default_rng(4712)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    x = bf(0.5 + 2.0 * rng.standard_normal((m, k)))
    g = bf(1.0 + 0.1 * rng.standard_normal(k))
    b = bf(0.1 * rng.standard_normal(k))
    W = bf(rng.standard_normal((n, k)) / np.sqrt(k))
    R, mu, rs = oracle.layernorm_linear(x, g, b, W, 1e-5)
    extra = ln_linear_extra(R, x, mu, rs, g, b, W)
    xd, gd, bd, Wd = (t.double().numpy() for t in (x, g, b, W))
    return dict(R=R, mu=mu, rs=rs, extra=extra, x=xd, g=gd, b=bd, W=Wd, k=k)


def _ln_kernel_like(c, Wf=None, drop_mean=False, drop_beta=False):
    # the epilogue form: fp32 x . Wf, c_n = sum Wf, d_n = sum beta W
    Wf = _bf16(c["W"] * c["g"][None, :]) if Wf is None else Wf
    acc = (c["x"].astype(np.float32) @ Wf.astype(np.float32).T).astype(np.float64)
    cn = Wf.astype(np.float32).sum(axis=1).astype(np.float64)
    dn = (c["W"].astype(np.float32) @ c["b"].astype(np.float32)).astype(np.float64)
    mu = 0.0 if drop_mean else c["mu"][:, None]
    d = 0.0 if drop_beta else dn[None, :]
    return _bf16(c["rs"][:, None] * (acc - mu * cn[None, :]) + d)


def test_ln_bound_admits_the_kernels_arithmetic(ln_case):
    check("emulated LN-linear", _ln_kernel_like(ln_case), ln_case["R"], "bf16", s=0.0,
          extra=ln_case["extra"])


@pytest.mark.parametrize("mistake", ["dropped K step", "mean not removed", "bias dropped",
                                     "coarser fold"])
def test_ln_bound_rejects_mistakes(ln_case, mistake):
    c = ln_case
    if mistake == "dropped K step":
        k0 = 16 * 9
        xc = (c["x"] - c["mu"][:, None]) * c["rs"][:, None] * c["g"][None, :] + c["b"][None, :]
        bad = _bf16(c["R"] - xc[:, k0:k0 + 16] @ c["W"][:, k0:k0 + 16].T)
    elif mistake == "mean not removed":
        bad = _ln_kernel_like(c, drop_mean=True)
    elif mistake == "bias dropped":
        bad = _ln_kernel_like(c, drop_beta=True)
    else:
        bad = _ln_kernel_like(c, Wf=_round_sig(c["W"] * c["g"][None, :], 4))
    with pytest.raises(AssertionError, match="outside the bound"):
        check(mistake, bad, c["R"], "bf16", s=0.0, extra=c["extra"])
