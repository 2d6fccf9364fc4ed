"""GPU parity of the RMSNorm -> linear fusion (rmsnorm_linear_fwd) against
the oracle's fp64 RMSNorm followed by an fp64 matrix product.

Bound, derived from the arithmetic: x enters the bf16 matrix cores exactly;
each product's weight w'_k W[n][k] is rounded once to bf16 (2^-9 relative)
and the K products are added in fp32 (at most K 2^-24 relative of their
magnitude sum), so |O - R| <= ulp_bf16(R) + 2^-8 S, S = sum_k |y_k W[n][k]|
(exact for w_norm NULL up to the fp32 sum), for K <= 65536."""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, to64, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_case(tag, m, n, k, seed, weight="w", gemma=False, rows=None):
    print(f"[case] {tag}: rmsnorm->linear M={m} N={n} K={k} weight={weight} gemma={gemma}",
          flush=True)
    x = workloads.normal((m, k), seed, torch.bfloat16)
    W = workloads.normal((n, k), seed + 1, torch.bfloat16, std=k ** -0.5)
    w = None if weight is None else workloads.normal(
        (k,), seed + 2, torch.bfloat16, mean=0.0 if gemma else 1.0, std=0.1)
    out, r = nr.rmsnorm_linear_fwd(x.to(DEV), None if w is None else w.to(DEV), W.to(DEV),
                                   1e-6, gemma)
    torch.cuda.synchronize()
    sel = np.arange(m) if rows is None else rows
    R, rr, S = oracle.rmsnorm_linear(x[sel], w, W, 1e-6, gemma)
    O = out.cpu()[sel]
    check(f"{tag} out", O, R, "bf16", s=0.0, extra=2.0 ** -8 * S)
    check(f"{tag} inv_rms", r.cpu()[sel], rr, "stat", s=0.0)
    # the bound is not vacuous: the error is far below the magnitude sum
    err = np.abs(to64(O) - R)
    assert np.max(err / (ulp_bf16(R) + 2.0 ** -8 * S)) <= 1.0
    return out


@pytest.mark.parametrize("m,n,k,weight,gemma", [
    (1, 128, 64, "w", False), (130, 256, 128, "w", True), (257, 384, 320, None, False),
    (1000, 1280, 5120, "w", False), (4096, 640, 5120, "w", True),
])
def test_rmsnorm_linear_cases(m, n, k, weight, gemma):
    run_case(f"{m}x{n}x{k}", m, n, k, 9800 + m + n + k, weight, gemma)


def test_rmsnorm_linear_long_sequence_sampled():
    m, n, k = 65536, 5120, 5120
    rng = np.random.default_rng(9900)
    rows = np.sort(rng.choice(m, 48, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 127, 128, m - 1]]))
    run_case("longseq", m, n, k, 9900, "w", False, rows=rows)


def test_rmsnorm_linear_matches_unfused_closely():
    # the fused and the unfused path (rmsnorm_fwd, then the vendor GEMM on
    # the bf16 y) each round once at the operand; both stay within the
    # oracle bound, and they agree with each other to the same order
    m, n, k = 512, 768, 1024
    x = workloads.normal((m, k), 9950, torch.bfloat16).to(DEV)
    w = workloads.normal((k,), 9951, torch.bfloat16, mean=1.0, std=0.1).to(DEV)
    W = workloads.normal((n, k), 9952, torch.bfloat16, std=k ** -0.5).to(DEV)
    out, r = nr.rmsnorm_linear_fwd(x, w, W)
    y, r2 = nr.rmsnorm_fwd(x, w, 1e-6)
    ref = (y.float() @ W.float().t())
    torch.cuda.synchronize()
    # the two sum x^2 in different orders: equal to a few fp32 ulps
    assert torch.allclose(r, r2, rtol=2e-6, atol=0)
    _, _, S = oracle.rmsnorm_linear(x.cpu(), w.cpu(), W.cpu())
    d = (out.float() - ref).abs().cpu().double().numpy()
    assert np.all(d <= ulp_bf16(ref.cpu().double().numpy()) + 2.0 ** -7 * S)
