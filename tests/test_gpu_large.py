"""GPU parity on tensors past 4 GiB: row and token addressing in 64 bits.

One bf16 activation of (2^20 + 3) rows x 4096 holds 4.3e9 elements (8.6 GB),
so byte offsets pass 2^32 and element offsets pass 2^31.  The inputs are drawn
on the device (seeded); sampled rows (the first, those around 2^19 and 2^20,
the last) are copied back and checked against the oracle element by element,
to the same bounds as every other parity test.  dW / dgamma / dbeta sum over
all rows and are checked at full size elsewhere, not here."""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, grad_scale

pytestmark = pytest.mark.gpu
DEV = "cuda"
ROWS, N = (1 << 20) + 3, 4096
SEL = np.array([0, 1, (1 << 19) - 1, 1 << 19, (1 << 20) - 1, 1 << 20, (1 << 20) + 1, (1 << 20) + 2])


@pytest.fixture(scope="module")
def big():
    print(f"[case] large tensors: {ROWS} x {N} bf16", flush=True)
    x = workloads.normal_device((ROWS, N), 9101, torch.bfloat16, DEV)
    dy = workloads.normal_device((ROWS, N), 9102, torch.bfloat16, DEV)
    w = workloads.normal((N,), 9103, torch.bfloat16, mean=1.0, std=0.1).to(DEV)
    b = workloads.normal((N,), 9104, torch.bfloat16, std=0.1).to(DEV)
    idx = torch.as_tensor(SEL, device=DEV)
    yield dict(x=x, dy=dy, w=w, b=b, idx=idx, xs=x[idx].cpu(), dys=dy[idx].cpu())
    torch.cuda.synchronize()


def test_rmsnorm_fwd_bwd_beyond_4gib(big):
    print("[case] rmsnorm fwd+bwd, 8.6 GB tensors", flush=True)
    x, dy, w, idx = big["x"], big["dy"], big["w"], big["idx"]
    y, r = nr.rmsnorm_fwd(x, w, 1e-6)
    dx, dw = nr.rmsnorm_bwd(dy, x, w, r)
    torch.cuda.synchronize()
    Y, R = oracle.rmsnorm_fwd(big["xs"], w.cpu(), 1e-6)
    DX, _ = oracle.rmsnorm_bwd(big["dys"], big["xs"], w.cpu(), 1e-6)
    check("y", y[idx].cpu(), Y, "bf16")
    check("inv_rms", r[idx].cpu(), R, "stat", s=0.0)
    check("dx", dx[idx].cpu(), DX, "bf16", s=grad_scale(R, big["dys"], w.cpu()))
    assert torch.isfinite(dw).all()
    del y, dx


def test_layernorm_fwd_bwd_beyond_4gib(big):
    print("[case] layernorm fwd+bwd, 8.6 GB tensors", flush=True)
    x, dy, w, b, idx = big["x"], big["dy"], big["w"], big["b"], big["idx"]
    y, mu, rs = nr.layernorm_fwd(x, w, b, 1e-5)
    dx, dg, db = nr.layernorm_bwd(dy, x, w, mu, rs)
    torch.cuda.synchronize()
    Y, MU, RS = oracle.layernorm_fwd(big["xs"], w.cpu(), b.cpu(), 1e-5)
    DX, _, _ = oracle.layernorm_bwd(big["dys"], big["xs"], w.cpu(), 1e-5)
    check("y", y[idx].cpu(), Y, "bf16")
    check("rstd", rs[idx].cpu(), RS, "stat", s=0.0)
    check("dx", dx[idx].cpu(), DX, "bf16", s=grad_scale(RS, big["dys"], w.cpu()))
    del y, dx


def test_fused_rmsnorm_rope_beyond_4gib(big):
    print("[case] fused rmsnorm -> rope fwd + bwd, 8.6 GB tensors, head_dim 128", flush=True)
    x, dy, w, idx = big["x"], big["dy"], big["w"], big["idx"]
    ct, st = nr.rope_table_1d(ROWS, 128, 0, 10000.0)
    y, r = nr.rmsnorm_rope_fwd(x, w, ct, st, 128)
    dx, dw = nr.rmsnorm_rope_bwd(dy, x, w, r, ct, st, 128)
    torch.cuda.synchronize()
    ang = oracle.rope_angles_1d(ROWS, 128, 0, 10000.0)[SEL]  # one row per token
    Y, R = oracle.rmsnorm_rope_fwd(big["xs"], w.cpu(), ang, 128)
    DX, _ = oracle.rmsnorm_rope_bwd(big["dys"], big["xs"], w.cpu(), ang, 128, want_dw=False)
    dy64 = oracle.rope_apply(big["dys"].view(1, len(SEL), N // 128, 128), ang,
                             inverse=True).reshape(len(SEL), N)
    check("y", y[idx].cpu(), Y, "bf16")
    check("inv_rms", r[idx].cpu(), R, "stat", s=0.0)
    check("dx", dx[idx].cpu(), DX, "bf16", s=grad_scale(R, dy64, w.cpu()))
    del y, dx


def test_layernorm_gelu_beyond_4gib(big):
    print("[case] layernorm + gelu fwd + bwd, 8.6 GB tensors", flush=True)
    x, dy, w, b, idx = big["x"], big["dy"], big["w"], big["b"], big["idx"]
    y, mu, rs = nr.layernorm_gelu_fwd(x, w, b, 1e-5)
    dx, dg, db = nr.layernorm_gelu_bwd(dy, x, w, b, mu, rs)
    torch.cuda.synchronize()
    Y, MU, RS = oracle.layernorm_gelu_fwd(big["xs"], w.cpu(), b.cpu(), 1e-5)
    DX, _, _ = oracle.layernorm_gelu_bwd(big["dys"], big["xs"], w.cpu(), b.cpu(), 1e-5,
                                         want_dw=False)
    check("y", y[idx].cpu(), Y, "bf16")
    check("rstd", rs[idx].cpu(), RS, "stat", s=0.0)
    # row scale of dx: the terms r * dout * gamma (|gelu'| stays below 1.13)
    check("dx", dx[idx].cpu(), DX, "bf16", s=1.13 * grad_scale(RS, big["dys"], w.cpu()))
    del y, dx


def test_rope_beyond_4gib(big):
    print("[case] rope forward then inverse, 8.6 GB tensor as [1, T, 32, 128]", flush=True)
    q = big["x"].clone().view(1, ROWS, N // 128, 128)
    ct, st = nr.rope_table_1d(ROWS, 128, 0, 10000.0)
    idx = big["idx"]
    nr.rope_interleaved_apply(q, ct, st)
    torch.cuda.synchronize()
    fwd_sel = q[0, idx].cpu()
    ang = oracle.rope_angles_1d(ROWS, 128, 0, 10000.0)[SEL]
    ref = oracle.rope_apply(big["xs"].view(1, len(SEL), N // 128, 128), ang)
    check("rope forward", fwd_sel, ref[0], "bf16")
    # the inverse is judged on the bytes it consumed: the forward's output
    nr.rope_interleaved_apply(q, ct, st, inverse=True)
    torch.cuda.synchronize()
    ref = oracle.rope_apply(fwd_sel.view(1, len(SEL), N // 128, 128), ang, inverse=True)
    check("rope inverse", q[0, idx].cpu(), ref[0], "bf16")
    del q
