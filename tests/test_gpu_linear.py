"""GPU parity of the RMSNorm -> linear fusion (rmsnorm_linear_fwd) against
the oracle's fp64 RMSNorm followed by an fp64 matrix product.

Bound, derived from the arithmetic (tolerance.linear_extra): x enters the
bf16 matrix cores exactly; each product's weight w'_k W[n][k] is rounded
once to bf16 and the K products are added in fp32, so
  |O - R| <= ulp_bf16(R) + 1e-5 |R| + c1 2^-9 sqrt(sum_k p_k^2) + c2 sqrt(K) 2^-24 S
with p_k = y_k W[n][k], S = sum_k |p_k|, c1 = 6 (0 without a norm weight,
W then entering exactly) and c2 = 8.  At K = 5120 with W ~ N(0, 1/K) that
is about 3 bf16 ulps of an output of size 1; numpy negative controls in
tests/test_oracle_linear.py show that a dropped 16-wide K step, a twice
applied norm weight and a coarser folded weight all break it.

Two kernels serve the call: 128 x 128 output tiles (small grids) and 256 x
256 tiles with the norm weight folded into W first (large grids); the tests
force each on the same shapes."""
import contextlib
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, linear_extra, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


@contextlib.contextmanager
def gemm_tile(tile):
    nr.nr_tune("gemm_tile", tile)
    try:
        yield
    finally:
        nr.nr_tune("gemm_tile", 0)


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
    idx = torch.as_tensor(sel, device=DEV)
    O = out[idx].cpu()
    y, _ = oracle.rmsnorm_fwd(x[sel], w, 1e-6, gemma)
    extra = linear_extra(R, y, W, folded=w is not None)
    worst = check(f"{tag} out", O, R, "bf16", s=0.0, extra=extra)
    check(f"{tag} inv_rms", r[idx].cpu(), rr, "stat", s=0.0)
    print(f"[case] {tag}: worst error / bound {worst:.3f}", flush=True)
    return out


@pytest.mark.parametrize("m,n,k,weight,gemma", [
    (1, 128, 64, "w", False), (130, 256, 128, "w", True), (257, 384, 320, None, False),
    (1000, 1280, 5120, "w", False), (4096, 640, 5120, "w", True),
])
def test_rmsnorm_linear_cases(m, n, k, weight, gemma):
    run_case(f"{m}x{n}x{k}", m, n, k, 9800 + m + n + k, weight, gemma)


@pytest.mark.parametrize("m,n,k,weight,gemma", [
    (1, 256, 64, "w", False), (777, 256, 5120, "w", False), (1000, 512, 320, "w", True),
    (300, 768, 192, None, False), (513, 1280, 1024, "w", False),
])
def test_rmsnorm_linear_tile256(m, n, k, weight, gemma):
    # the 256 x 256 kernel on small shapes: ragged M (rows past M read out of
    # range), an odd number of K steps (320 = 5 x 64), a single row
    with gemm_tile(2):
        run_case(f"tile256 {m}x{n}x{k}", m, n, k, 9700 + m + n + k, weight, gemma)


@pytest.mark.parametrize("tile", [1, 2])
def test_rmsnorm_linear_folded_weight_is_bit_identical(tile):
    # rmsnorm_linear_fold_weight, then a call without norm weight, gives the
    # same bits as the call with it (one rounding of w' W either way)
    print(f"[case] folded weight, tile {tile}", flush=True)
    m, n, k = 600, 512, 448
    x = workloads.normal((m, k), 9960, torch.bfloat16).to(DEV)
    w = workloads.normal((k,), 9961, torch.bfloat16, mean=0.0, std=0.1).to(DEV)
    W = workloads.normal((n, k), 9962, torch.bfloat16, std=k ** -0.5).to(DEV)
    with gemm_tile(tile):
        a, ra = nr.rmsnorm_linear_fwd(x, w, W, 1e-6, True)
        Wf = nr.rmsnorm_linear_fold_weight(w, W, True)
        b, rb = nr.rmsnorm_linear_fwd(x, None, Wf, 1e-6)
        # the fold in place gives the same folded weight
        W2 = W.clone()
        nr.rmsnorm_linear_fold_weight(w, W2, True, out=W2)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(ra, rb)
    assert torch.equal(W2, Wf)
    ref = (W.float() * (1.0 + w.float())).to(torch.bfloat16)  # one rounding of an exact product
    assert torch.equal(Wf, ref)


def test_rmsnorm_linear_tiles_agree_and_workspace_is_reused():
    # both kernels on one shape: each within the oracle bound (run_case), and
    # close to each other (their x^2 sums run in different orders); a caller
    # workspace serves repeated calls
    print("[case] tile 128 vs 256, 1024x1024x2048", flush=True)
    m, n, k = 1024, 1024, 2048
    x = workloads.normal((m, k), 9970, torch.bfloat16).to(DEV)
    w = workloads.normal((k,), 9971, torch.bfloat16, mean=1.0, std=0.1).to(DEV)
    W = workloads.normal((n, k), 9972, torch.bfloat16, std=k ** -0.5).to(DEV)
    with gemm_tile(1):
        a, ra = nr.rmsnorm_linear_fwd(x, w, W)
    with gemm_tile(2):
        ws = torch.empty(nr.nr_rmsnorm_linear_workspace_bytes(m, n, k, True), dtype=torch.uint8,
                         device=DEV)
        assert ws.numel() == m * 4 + n * k * 2
        b, rb = nr.rmsnorm_linear_fwd(x, w, W, workspace=ws)
        c, rc = nr.rmsnorm_linear_fwd(x, w, W, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(b, c) and torch.equal(rb, rc)
    assert torch.allclose(ra, rb, rtol=2e-6, atol=0)
    d = (a.float() - b.float()).abs().cpu().double().numpy()
    assert np.all(d <= 2 * ulp_bf16(a.float().cpu().double().numpy()) + 1e-6)


@pytest.mark.parametrize("tile", [1, 2])
def test_rmsnorm_linear_widest_n(tile):
    # N = 2^22, the largest accepted: within a row tile the output's byte
    # offsets reach 2^31 - 16, the end of the 32-bit buffer range
    m, n, k = 300, 1 << 22, 64
    with gemm_tile(tile):
        run_case(f"widest N, tile {tile}", m, n, k, 9980 + tile, "w", False,
                 rows=np.array([0, 1, 127, 128, 255, 256, 299]))


@pytest.mark.parametrize("tile", [1, 2])
def test_rmsnorm_linear_longest_k(tile):
    # K = 65536, the largest accepted: 1024 K steps, operand offsets of a
    # 256-row tile up to 32 MiB
    m, n, k = 300, 256, 65536
    with gemm_tile(tile):
        run_case(f"longest K, tile {tile}", m, n, k, 9990 + tile, "w", True,
                 rows=np.array([0, 1, 100, 255, 256, 299]))


def test_rmsnorm_linear_long_sequence_sampled():
    m, n, k = 65536, 5120, 5120
    rng = np.random.default_rng(9900)
    rows = np.sort(rng.choice(m, 48, replace=False))
    rows = np.unique(np.concatenate([rows, [0, 127, 128, m - 1]]))
    run_case("longseq", m, n, k, 9900, "w", False, rows=rows)


def test_rmsnorm_linear_matches_unfused_closely():
    # the fused and the unfused path (rmsnorm_fwd, then the vendor GEMM on
    # the bf16 y) each round once at the operand
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
    # both are held to the same derived bound of the fp64 composition (the
    # unfused path rounds y to bf16 where the fused one rounds w' W)
    R, _, _ = oracle.rmsnorm_linear(x.cpu(), w.cpu(), W.cpu())
    y64, _ = oracle.rmsnorm_fwd(x.cpu(), w.cpu(), 1e-6)
    extra = linear_extra(R, y64, W.cpu(), folded=True)
    check("fused", out.cpu(), R, "bf16", s=0.0, extra=extra)
    check("unfused", ref.cpu(), R, "bf16", s=0.0, extra=extra)


# ---- LayerNorm -> linear (layernorm_linear_fwd) -------------------------------
#
# Against the oracle's fp64 LayerNorm followed by the fp64 product, within
# tolerance.ln_linear_extra (derived from the folded weight's rounding, the
# fp32 sums of the product and of the column terms, and the statistics).

from tolerance import ln_linear_extra  # noqa: E402


def run_ln_case(tag, m, n, k, seed, affine=("g", "b"), mean=0.5, std=2.0, rows=None):
    print(f"[case] {tag}: layernorm->linear M={m} N={n} K={k} affine={affine}", flush=True)
    x = workloads.normal((m, k), seed, torch.bfloat16, mean=mean, std=std)
    W = workloads.normal((n, k), seed + 1, torch.bfloat16, std=k ** -0.5)
    g = workloads.normal((k,), seed + 2, torch.bfloat16, mean=1.0, std=0.1) if "g" in affine else None
    b = workloads.normal((k,), seed + 3, torch.bfloat16, std=0.1) if "b" in affine else None
    dv = lambda t: None if t is None else t.to(DEV)
    out, mu, rs = nr.layernorm_linear_fwd(x.to(DEV), dv(g), dv(b), W.to(DEV), 1e-5)
    torch.cuda.synchronize()
    sel = np.arange(m) if rows is None else rows
    R, rmu, rrs = oracle.layernorm_linear(x[sel], g, b, W, 1e-5)
    idx = torch.as_tensor(sel, device=DEV)
    extra = ln_linear_extra(R, x[sel], rmu, rrs, g, b, W)
    worst = check(f"{tag} out", out[idx].cpu(), R, "bf16", s=0.0, extra=extra)
    x64 = x[sel].double().numpy()
    check(f"{tag} mean", mu[idx].cpu(), rmu, "stat", s=np.sqrt(np.mean(x64 * x64, axis=1)))
    check(f"{tag} rstd", rs[idx].cpu(), rrs, "stat", s=0.0)
    print(f"[case] {tag}: worst error / bound {worst:.3f}", flush=True)


@pytest.mark.parametrize("m,n,k,affine", [
    (1, 256, 64, ("g", "b")), (130, 256, 128, ()), (257, 512, 320, ("g",)),
    (1000, 1280, 5120, ("g", "b")), (4096, 768, 5120, ("b",)),
    # rows held in 10 and 16 chunks per lane by the statistics pass, and past
    # that (read twice; K = 65536 below)
    (200, 256, 3072, ()), (70, 256, 8192, ("g", "b")), (33, 256, 8256, ("g",)),
])
def test_layernorm_linear_cases(m, n, k, affine):
    run_ln_case(f"ln {m}x{n}x{k}", m, n, k, 9600 + m + n + k, affine)


def test_layernorm_linear_large_mean_rows():
    # rows whose mean is four times their spread: the mean is removed after
    # the product, so the bound carries the uncentred magnitude sum
    run_ln_case("ln large mean", 600, 512, 2048, 9610, mean=4.0, std=1.0)


def test_layernorm_linear_widest_n_and_longest_k():
    run_ln_case("ln widest N", 300, 1 << 22, 64, 9620, rows=np.array([0, 1, 255, 256, 299]))
    run_ln_case("ln longest K", 300, 256, 65536, 9630, rows=np.array([0, 1, 100, 255, 256, 299]))


def test_layernorm_linear_long_sequence_sampled():
    m, n, k = 65536, 5120, 5120
    rng = np.random.default_rng(9640)
    rows = np.unique(np.concatenate([rng.choice(m, 48, replace=False), [0, 255, 256, m - 1]]))
    run_ln_case("ln longseq", m, n, k, 9640, rows=rows)


def test_layernorm_linear_stats_to_workspace_and_reuse():
    # without caller statistics the workspace takes them; a caller workspace
    # serves repeated calls with identical results
    print("[case] ln->linear: statistics in the workspace, workspace reused", flush=True)
    m, n, k = 700, 512, 1024
    x = workloads.normal((m, k), 9650, torch.bfloat16, mean=0.5, std=2.0).to(DEV)
    W = workloads.normal((n, k), 9651, torch.bfloat16, std=k ** -0.5).to(DEV)
    g = workloads.normal((k,), 9652, torch.bfloat16, mean=1.0, std=0.1).to(DEV)
    b = workloads.normal((k,), 9653, torch.bfloat16, std=0.1).to(DEV)
    ws = torch.empty(nr.nr_layernorm_linear_workspace_bytes(m, n, k, True), dtype=torch.uint8,
                     device=DEV)
    a, mu, rs = nr.layernorm_linear_fwd(x, g, b, W, workspace=ws)
    c, _, _ = nr.layernorm_linear_fwd(x, g, b, W, want_stats=False, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, c)
