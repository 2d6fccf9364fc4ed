"""GPU checks of the PyTorch layer: its autograd Functions and modules call
the C ABI and give the oracle's results (to the same bounds as the direct
calls), a swapped-in model computes what the original model computes, and
ten training steps through the fused modules follow an fp64 CPU model whose
norms are the oracle's (the write-up's same-weights training comparison,
"Helios 性能优化全解析", 内核二 FlashRoPE: each kernel file ends with a gradient
check and a ten-step same-weights training comparison)."""
import copy

import numpy as np
import pytest
import torch
from torch import nn

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from rmsnorm_layernorm_fwd_amd import layers as L
from tolerance import check, grad_scale, out_kind, to64, ulp_bf16, ulp_f16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[case] {msg}", flush=True)


def param_grad_check(name, o, r, dtype):
    """A weight gradient: fp32 from the kernel, then rounded to the
    parameter's dtype (one more rounding for bf16 and fp16)."""
    extra = {torch.bfloat16: ulp_bf16, torch.float16: ulp_f16}.get(dtype)
    extra = None if extra is None else extra(to64(r))
    check(name, o, r, "col", extra=extra)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("gemma", [False, True])
def test_rms_module(dtype, gemma):
    say(f"FlashRMSNorm {dtype} gemma={gemma}")
    seed = 9100 + int(gemma)
    x = workloads.normal((3, 37, 320), seed, dtype)
    w = workloads.normal((320,), seed + 1, dtype, mean=0.0 if gemma else 1.0, std=0.1)
    dout = workloads.normal((3, 37, 320), seed + 2, dtype)
    m = L.FlashRMSNorm(320, eps=1e-6, gemma=gemma, device=DEV, dtype=dtype)
    with torch.no_grad():
        m.weight.copy_(w.to(DEV))
    xg = x.to(DEV).requires_grad_(True)
    y = m(xg)
    y.backward(dout.to(DEV))
    torch.cuda.synchronize()
    ry, rr = oracle.rmsnorm_fwd(x, w, 1e-6, gemma)
    rdx, rdw = oracle.rmsnorm_bwd(dout, x, w, 1e-6, gemma)
    k = out_kind(dtype)
    check("y", y.reshape(-1, 320), ry, k)
    check("dx", xg.grad.reshape(-1, 320), rdx, k,
          s=grad_scale(rr, dout.reshape(-1, 320), w, gemma))
    param_grad_check("dw", m.weight.grad, rdw, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("affine", [True, False])
def test_layernorm_modules(dtype, gelu, affine):
    say(f"FlashLayerNorm{'Gelu' if gelu else ''} {dtype} affine={affine}")
    seed = 9200 + 2 * int(gelu) + int(affine)
    n = 264
    x = workloads.normal((5, 11, n), seed, dtype, mean=0.5, std=2.0)
    gm = workloads.normal((n,), seed + 1, dtype, mean=1.0, std=0.1) if affine else None
    bt = workloads.normal((n,), seed + 2, dtype, std=0.2) if affine else None
    dout = workloads.normal((5, 11, n), seed + 3, dtype)
    cls = L.FlashLayerNormGelu if gelu else L.FlashLayerNorm
    m = cls(n, eps=1e-5, elementwise_affine=affine, device=DEV, dtype=dtype)
    if affine:
        with torch.no_grad():
            m.weight.copy_(gm.to(DEV))
            m.bias.copy_(bt.to(DEV))
    xg = x.to(DEV).requires_grad_(True)
    y = m(xg)
    y.backward(dout.to(DEV))
    torch.cuda.synchronize()
    x2, d2 = x.reshape(-1, n), dout.reshape(-1, n)
    if gelu:
        ry, _, rrs = oracle.layernorm_gelu_fwd(x2, gm, bt, 1e-5)
        rdx, rdg, rdb = oracle.layernorm_gelu_bwd(d2, x2, gm, bt, 1e-5)
        scale = 1.13 * grad_scale(rrs, d2, gm)
    else:
        ry, _, rrs = oracle.layernorm_fwd(x2, gm, bt, 1e-5)
        rdx, rdg, rdb = oracle.layernorm_bwd(d2, x2, gm, 1e-5)
        scale = grad_scale(rrs, d2, gm)
    k = out_kind(dtype)
    check("y", y.reshape(-1, n), ry, k)
    check("dx", xg.grad.reshape(-1, n), rdx, k, s=scale)
    if affine:
        param_grad_check("dgamma", m.weight.grad, rdg, dtype)
        param_grad_check("dbeta", m.bias.grad, rdb, dtype)


@pytest.mark.parametrize("gelu", [False, True])
def test_fp32_parameters_with_bf16_activations(gelu):
    # mixed precision: the module's fp32 parameters are cast to the input's
    # bf16 for the kernel; the output equals that of a module holding the
    # rounded parameters, and the parameters' gradients come back in fp32,
    # straight from the kernel's fp32 sums (the bf16 module rounds them)
    say(f"fp32 parameters, bf16 input, {'LayerNorm+GeLU' if gelu else 'RMSNorm / LayerNorm'}")
    n = 256
    x = workloads.normal((7, n), 9300, torch.bfloat16).to(DEV)
    dout = workloads.normal((7, n), 9301, torch.bfloat16).to(DEV)
    w32 = workloads.normal((n,), 9302, torch.float32, mean=1.0, std=0.1).to(DEV)
    b32 = workloads.normal((n,), 9303, torch.float32, std=0.1).to(DEV)
    pairs = [(L.FlashRMSNorm(n, device=DEV), L.FlashRMSNorm(n, device=DEV, dtype=torch.bfloat16))]
    cls = L.FlashLayerNormGelu if gelu else L.FlashLayerNorm
    pairs.append((cls(n, device=DEV), cls(n, device=DEV, dtype=torch.bfloat16)))
    for m32, m16 in pairs:
        with torch.no_grad():
            m32.weight.copy_(w32)
            m16.weight.copy_(w32.to(torch.bfloat16))
            if getattr(m32, "bias", None) is not None:
                m32.bias.copy_(b32)
                m16.bias.copy_(b32.to(torch.bfloat16))
        xa, xb = x.clone().requires_grad_(True), x.clone().requires_grad_(True)
        ya, yb = m32(xa), m16(xb)
        ya.backward(dout)
        yb.backward(dout)
        torch.cuda.synchronize()
        assert ya.dtype == torch.bfloat16 and torch.equal(ya, yb)
        assert torch.equal(xa.grad, xb.grad)
        assert m32.weight.grad.dtype == torch.float32
        assert torch.equal(m32.weight.grad.to(torch.bfloat16), m16.weight.grad)
        assert not torch.equal(m32.weight.grad, m16.weight.grad.float())  # not rounded


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("inplace", [False, True])
def test_rope_function(dtype, inplace):
    say(f"apply_rotary_emb_interleaved {dtype} inplace={inplace}")
    b, t, h, d = 2, 19, 3, 64
    x = workloads.normal((b, t, h, d), 9300 + int(inplace), dtype)
    dout = workloads.normal((b, t, h, d), 9302, dtype)
    ang = oracle.rope_angles_1d(t, d, 0, 10000.0)
    ct, st = nr.rope_table_1d(t, d, 0, 10000.0)
    leaf = x.to(DEV).requires_grad_(True)
    src = leaf * 1 if inplace else leaf  # in place needs a non-leaf
    y = L.apply_rotary_emb_interleaved(src, ct, st, inplace=inplace)
    y.backward(dout.to(DEV))
    torch.cuda.synchronize()
    k = out_kind(dtype)
    check("rope y", y.reshape(-1, d), oracle.rope_apply(x, ang).reshape(-1, d), k)
    check("rope dx", leaf.grad.reshape(-1, d),
          oracle.rope_apply(dout, ang, inverse=True).reshape(-1, d), k)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rms_norm_rope_function(per_head, dtype):
    say(f"rms_norm_rope per_head={per_head} {dtype}")
    b, t, h, d = 2, 13, 4, 32
    n = d if per_head else h * d
    x = workloads.normal((b, t, h, d), 9400 + int(per_head), dtype)
    w = workloads.normal((n,), 9402, dtype, mean=1.0, std=0.1)
    dout = workloads.normal((b, t, h, d), 9403, dtype)
    ct, st = nr.rope_table_1d(t, d, 0, 10000.0)
    wp = w.to(DEV).requires_grad_(True)
    xg = x.to(DEV).requires_grad_(True)
    y = L.rms_norm_rope(xg, wp, ct, st, eps=1e-6, per_head=per_head)
    y.backward(dout.to(DEV))
    torch.cuda.synchronize()
    ang = np.tile(oracle.rope_angles_1d(t, d, 0, 10000.0), (b, 1))  # table row per (b, t)
    rpt = h if per_head else 1
    x2, d2 = x.reshape(-1, n), dout.reshape(-1, n)
    ry, rr = oracle.rmsnorm_rope_fwd(x2, w, ang, d, rpt, 1e-6)
    rdx, rdw = oracle.rmsnorm_rope_bwd(d2, x2, w, ang, d, rpt, 1e-6)
    k = out_kind(dtype)
    check("y", y.reshape(-1, n), ry, k)
    rdy = oracle.rope_apply(d2.reshape(1, -1, n // d, d), np.repeat(ang, rpt, axis=0)
                            if per_head else ang, inverse=True).reshape(-1, n)
    check("dx", xg.grad.reshape(-1, n), rdx, k, s=grad_scale(rr, rdy, w))
    param_grad_check("dw", wp.grad, rdw, dtype)


class MyRMSNorm(nn.Module):
    """An RMSNorm as models define it (plain PyTorch)."""

    def __init__(self, n, eps):
        super().__init__()
        self.weight = nn.Parameter(torch.ones(n))
        self.variance_epsilon = eps

    def forward(self, x):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.variance_epsilon) * self.weight


class GemmaRMSNorm(MyRMSNorm):
    def forward(self, x):
        return x * torch.rsqrt(x.pow(2).mean(-1, keepdim=True) + self.variance_epsilon) * (1 + self.weight)


def small_model(seed):
    torch.manual_seed(seed)
    m = nn.Sequential(nn.Linear(96, 96), nn.LayerNorm(96), nn.Linear(96, 96), MyRMSNorm(96, 1e-6),
                      nn.Linear(96, 96), GemmaRMSNorm(96, 1e-6), nn.RMSNorm(96, eps=1e-5))
    with torch.no_grad():
        for mod in m.modules():
            w = getattr(mod, "weight", None)
            if w is not None and w.dim() == 1:
                w.add_(0.1 * torch.randn_like(w))
            b = getattr(mod, "bias", None)
            if isinstance(mod, nn.LayerNorm) and b is not None:
                b.add_(0.1 * torch.randn_like(b))
    return m


def test_replace_all_norms_keeps_the_model_output():
    say("replace_all_norms_with_flash_norms on a small model")
    ref = small_model(7).double()
    m = copy.deepcopy(ref).float().to(DEV)
    assert L.replace_all_norms_with_flash_norms(m) == 4
    x = workloads.normal((6, 17, 96), 9500, torch.float32)
    with torch.no_grad():
        want = ref(x.double())
        got = m(x.to(DEV))
    torch.cuda.synchronize()
    # fp32 kernels and fp32 GEMMs against the same model in fp64
    check("patched model", got.reshape(-1, 96), want.reshape(-1, 96), "f32",
          extra=1e-5 * np.abs(to64(want.reshape(-1, 96))).max())


class OracleRMS(torch.autograd.Function):
    """RMSNorm whose forward and backward are the oracle's (fp64, CPU)."""

    @staticmethod
    def forward(ctx, x, w, eps):
        ctx.save_for_backward(x, w)
        ctx.eps = eps
        y, _ = oracle.rmsnorm_fwd(x.detach(), w.detach(), eps)
        return torch.from_numpy(y).view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        dx, dw = oracle.rmsnorm_bwd(dy.contiguous(), x.detach(), w.detach(), ctx.eps)
        return torch.from_numpy(dx).view(x.shape), torch.from_numpy(dw), None


class OracleLN(torch.autograd.Function):
    """LayerNorm whose forward and backward are the oracle's (fp64, CPU)."""

    @staticmethod
    def forward(ctx, x, g, b, eps):
        ctx.save_for_backward(x, g)
        ctx.eps = eps
        y, _, _ = oracle.layernorm_fwd(x.detach(), g.detach(), b.detach(), eps)
        return torch.from_numpy(y).view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x, g = ctx.saved_tensors
        dx, dg, db = oracle.layernorm_bwd(dy.contiguous(), x.detach(), g.detach(), ctx.eps)
        return torch.from_numpy(dx).view(x.shape), torch.from_numpy(dg), torch.from_numpy(db), None


def test_ten_training_steps_follow_the_oracle():
    say("10 SGD steps: fused modules on the GPU vs oracle norms in fp64 on the CPU")
    torch.manual_seed(11)
    lin = [nn.Linear(128, 128) for _ in range(3)]
    rms_w = nn.Parameter(1 + 0.1 * torch.randn(128))
    ln_g = nn.Parameter(1 + 0.1 * torch.randn(128))
    ln_b = nn.Parameter(0.1 * torch.randn(128))
    x = workloads.normal((8, 64, 128), 9600, torch.float32)
    target = workloads.normal((8, 64, 128), 9601, torch.float32)

    # GPU: fp32 parameters, the fused modules
    g_lin = [copy.deepcopy(m).to(DEV) for m in lin]
    g_rms = L.FlashRMSNorm(128, eps=1e-6, device=DEV)
    g_ln = L.FlashLayerNorm(128, eps=1e-5, device=DEV)
    with torch.no_grad():
        g_rms.weight.copy_(rms_w)
        g_ln.weight.copy_(ln_g)
        g_ln.bias.copy_(ln_b)
    g_params = [p for m in g_lin for p in m.parameters()] + [g_rms.weight, g_ln.weight, g_ln.bias]

    # CPU: fp64 copies, norms through the oracle
    c_lin = [copy.deepcopy(m).double() for m in lin]
    c_rms_w = nn.Parameter(rms_w.detach().double().clone())
    c_ln_g = nn.Parameter(ln_g.detach().double().clone())
    c_ln_b = nn.Parameter(ln_b.detach().double().clone())
    c_params = [p for m in c_lin for p in m.parameters()] + [c_rms_w, c_ln_g, c_ln_b]

    def g_fwd(inp):
        h = g_rms(g_lin[0](inp))
        h = g_ln(g_lin[1](torch.tanh(h)))
        return g_lin[2](h)

    def c_fwd(inp):
        h = OracleRMS.apply(c_lin[0](inp), c_rms_w, 1e-6)
        h = OracleLN.apply(c_lin[1](torch.tanh(h)), c_ln_g, c_ln_b, 1e-5)
        return c_lin[2](h)

    xg, tg = x.to(DEV), target.to(DEV)
    xc, tc = x.double(), target.double()
    lr = 0.05
    g_losses, c_losses = [], []
    for _ in range(10):
        for ps in (g_params, c_params):
            for p in ps:
                p.grad = None
        lg = ((g_fwd(xg) - tg) ** 2).mean()
        lc = ((c_fwd(xc) - tc) ** 2).mean()
        lg.backward()
        lc.backward()
        with torch.no_grad():
            for p in g_params:
                p -= lr * p.grad
            for p in c_params:
                p -= lr * p.grad
        g_losses.append(float(lg.detach()))
        c_losses.append(float(lc.detach()))
    torch.cuda.synchronize()
    say(f"losses gpu {g_losses[0]:.6f}..{g_losses[-1]:.6f} cpu {c_losses[0]:.6f}..{c_losses[-1]:.6f}")
    assert g_losses[-1] < g_losses[0]  # it trains
    # fp32 end to end (GEMMs included) against fp64: agreement to ~1e-5
    np.testing.assert_allclose(g_losses, c_losses, rtol=2e-5)
    for pg, pc in zip(g_params, c_params):
        check("trained parameter", pg.reshape(1, -1), pc.detach().reshape(1, -1), "f32",
              extra=2e-5 * np.abs(to64(pc)).max())
