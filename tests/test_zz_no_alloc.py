"""GPU check of rmsnorm_bwd_noalloc, the backward for callers that cannot
allocate: through the C ABI, two calls in a row (the second on a smaller
batch and shorter rows, so the shared scratch array holds the first call's
partial rows when the second starts), each against rmsnorm_bwd with a
caller workspace (the same kernels: the same bits) and against the fp64
oracle within the usual bounds."""
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, grad_scale

pytestmark = pytest.mark.gpu
DEV = "cuda"


def one_call(rows, n, seed, gemma):
    print(f"[case] rmsnorm_bwd_noalloc {rows}x{n} bf16 gemma={gemma}", flush=True)
    x = workloads.normal((rows, n), seed, torch.bfloat16)
    w = workloads.normal((n,), seed + 1, torch.bfloat16, mean=0.0 if gemma else 1.0, std=0.1)
    dy = workloads.normal((rows, n), seed + 2, torch.bfloat16)
    xg, wg, dyg = x.to(DEV), w.to(DEV), dy.to(DEV)
    _, r = nr.rmsnorm_fwd(xg, wg, 1e-6, gemma)
    dx_ref, dw_ref = nr.rmsnorm_bwd(dyg, xg, wg, r, gemma)
    dx = torch.full_like(xg, 7.0)
    dw = torch.full((n,), 7.0, dtype=torch.float32, device=DEV)
    nr.rmsnorm_bwd_noalloc(dyg, xg, wg, r, dx, dw, gemma)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref), "dx differs from rmsnorm_bwd"
    assert torch.equal(dw, dw_ref), "dw differs from rmsnorm_bwd"
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, 1e-6, gemma)
    _, rr = oracle.rmsnorm_fwd(x, w, 1e-6, gemma)
    check("noalloc dx", dx.cpu(), rdx, "bf16", s=grad_scale(rr, dy, w, gemma))
    check("noalloc dw", dw.cpu(), rdw, "col")


def test_noalloc_matches_workspace_call_twice_second_smaller():
    one_call(8192, 5120, 7100, False)
    one_call(1000, 3000, 7200, True)


def test_noalloc_per_head_rows_twice_second_smaller():
    # rows of at most 32 chunks: the packed backward's partial rows in the
    # scratch array (up to 1280 of them), then a smaller batch of wider rows
    one_call(90000, 128, 7300, False)
    one_call(5000, 256, 7400, True)


def test_noalloc_without_dw_and_empty_batch():
    print("[case] rmsnorm_bwd_noalloc without dw; empty batch", flush=True)
    x = workloads.normal((300, 640), 7300, torch.bfloat16).to(DEV)
    w = torch.ones(640, dtype=torch.bfloat16, device=DEV)
    dy = workloads.normal((300, 640), 7301, torch.bfloat16).to(DEV)
    _, r = nr.rmsnorm_fwd(x, w)
    dx_ref, _ = nr.rmsnorm_bwd(dy, x, w, r, want_dw=False)
    dx = torch.empty_like(x)
    nr.rmsnorm_bwd_noalloc(dy, x, w, r, dx, None)
    e = torch.empty(0, 640, dtype=torch.bfloat16, device=DEV)
    dw0 = torch.full((640,), 3.0, dtype=torch.float32, device=DEV)
    nr.rmsnorm_bwd_noalloc(e, e, w, torch.empty(0, device=DEV), torch.empty_like(e), dw0)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_ref)
    assert int(dw0.count_nonzero()) == 0  # a sum over no rows


def test_noalloc_long_rows_twice_second_smaller():
    # rows over 16384 elements: the two-pass backward (65536), whose partial
    # rows and row terms both live in the scratch array, then the one-pass
    # backward with its accumulators in LDS (20000 bf16); a workspace beyond
    # the array, millions of such rows, is refused on the host (ABI test)
    one_call(512, 65536, 7400, False)
    one_call(100, 20000, 7500, True)
