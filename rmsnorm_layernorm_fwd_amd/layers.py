"""PyTorch-facing layer over the C ABI: autograd Functions, drop-in modules
and model patch functions.

The write-up this library follows ("Helios 性能优化全解析", sections 内核全景
and 如何启用) ships its kernels as patch functions that swap a model's norm
modules and its RoPE helper without changing the model's interface, and an
autograd Function whose backward is the forward kernel with sin negated
(内核二 FlashRoPE).  This module offers the same shape of interface:

* functional ops with autograd: ``rms_norm``, ``layer_norm``,
  ``layer_norm_gelu``, ``rms_norm_rope``, ``apply_rotary_emb_interleaved``;
* modules: ``FlashRMSNorm``, ``FlashLayerNorm``, ``FlashLayerNormGelu``;
* patches: ``replace_all_norms_with_flash_norms``,
  ``replace_rmsnorm_with_fp32``, ``replace_rope_with_flash_rope``.

Every forward and backward runs in the HIP kernels through the binding in
this package; there is no PyTorch or CPU fallback (a CPU tensor raises).
Weight gradients come out of the kernels in fp32 and are cast to the
parameter's dtype, as autograd requires.
"""
from __future__ import annotations

import torch
from torch import nn

from . import (layernorm_bwd, layernorm_fwd, layernorm_gelu_bwd, layernorm_gelu_fwd,
               rmsnorm_bwd, rmsnorm_fwd, rmsnorm_rope_bwd, rmsnorm_rope_fwd,
               rope_interleaved_apply)

__all__ = [
    "rms_norm", "layer_norm", "layer_norm_gelu", "rms_norm_rope", "apply_rotary_emb_interleaved",
    "rope_tables", "FlashRMSNorm", "FlashLayerNorm", "FlashLayerNormGelu",
    "replace_all_norms_with_flash_norms", "replace_rmsnorm_with_fp32",
    "replace_rope_with_flash_rope",
]


def _rows(t: torch.Tensor) -> torch.Tensor:
    """[..., n] -> contiguous [rows, n] (a view when already contiguous)."""
    return t.contiguous().view(-1, t.shape[-1])


def _grad_rows(g: torch.Tensor, like: torch.Tensor) -> torch.Tensor:
    if g.dtype != like.dtype:
        g = g.to(like.dtype)
    return _rows(g)


def _param_grad(g, dtype):
    """A weight gradient: fp32 from the kernel, returned in the parameter's
    own dtype (no rounding for an fp32 parameter)."""
    return None if g is None or dtype is None else g.to(dtype)


def _as_input_dtype(p, x):
    """The kernels take weights in the input's storage type: a parameter of
    another dtype (fp32 master weights under bf16 activations) is cast for
    the kernel, rounding it once; its gradient is still returned in the
    parameter's dtype, straight from the kernel's fp32 sums."""
    return p if p is None or p.dtype == x.dtype else p.to(x.dtype)


def _dtype(p):
    return None if p is None else p.dtype


# ---------------------------------------------------------------- RMSNorm

class _RMSNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, weight, eps, gemma):
        x2 = _rows(x)
        wk = _as_input_dtype(weight, x)
        y, r = rmsnorm_fwd(x2, wk, eps, gemma)
        ctx.save_for_backward(x2, wk, r)
        ctx.gemma, ctx.wdt = gemma, _dtype(weight)
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, weight, r = ctx.saved_tensors
        want_dw = weight is not None and ctx.needs_input_grad[1]
        dx, dw = rmsnorm_bwd(_grad_rows(dy, x2), x2, weight, r, ctx.gemma, want_dw=want_dw)
        return dx.view(dy.shape), _param_grad(dw, ctx.wdt), None, None


def rms_norm(x, weight=None, eps=1e-6, gemma=False):
    """y = x / sqrt(mean(x^2) + eps) * w' over the last axis (w' = w, 1 + w
    with ``gemma``, or 1 without a weight); fp32 arithmetic, one rounding."""
    return _RMSNormFn.apply(x, weight, float(eps), bool(gemma))


# ---------------------------------------------------------------- LayerNorm

class _LayerNormFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, gamma, beta, eps, gelu):
        x2 = _rows(x)
        gk, bk = _as_input_dtype(gamma, x), _as_input_dtype(beta, x)
        fwd = layernorm_gelu_fwd if gelu else layernorm_fwd
        y, mu, rs = fwd(x2, gk, bk, eps)
        ctx.save_for_backward(x2, gk, bk, mu, rs)
        ctx.gelu, ctx.gdt, ctx.bdt = gelu, _dtype(gamma), _dtype(beta)
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, dy):
        x2, gamma, beta, mu, rs = ctx.saved_tensors
        want_g = gamma is not None and ctx.needs_input_grad[1]
        want_b = beta is not None and ctx.needs_input_grad[2]
        g2 = _grad_rows(dy, x2)
        if ctx.gelu:
            dx, dg, db = layernorm_gelu_bwd(g2, x2, gamma, beta, mu, rs, want_dgamma=want_g,
                                            want_dbeta=want_b)
        else:
            dx, dg, db = layernorm_bwd(g2, x2, gamma, mu, rs, want_dgamma=want_g,
                                       want_dbeta=want_b)
        return dx.view(dy.shape), _param_grad(dg, ctx.gdt), _param_grad(db, ctx.bdt), None, None


def layer_norm(x, weight=None, bias=None, eps=1e-5):
    """y = (x - mean) / sqrt(var + eps) * weight + bias over the last axis
    (biased variance); fp32 arithmetic, one rounding."""
    return _LayerNormFn.apply(x, weight, bias, float(eps), False)


def layer_norm_gelu(x, weight=None, bias=None, eps=1e-5):
    """gelu_tanh(layer_norm(x)) in one pass each way."""
    return _LayerNormFn.apply(x, weight, bias, float(eps), True)


# ---------------------------------------------------------------- RoPE

def rope_tables(cos, sin=None):
    """Normalise a caller's rotary tables to the kernels' per-pair fp32
    layout [tokens, head_dim/2].

    Accepts per-pair tables, tables duplicated over the interleaved pair
    ([tokens, head_dim], entry 2i == entry 2i+1: the even columns are
    taken), or one complex tensor e^{i angle} [tokens, head_dim/2] as ``cos``
    with ``sin`` None.  Extra leading axes of size 1 are dropped."""
    if sin is None:
        if not torch.is_complex(cos):
            raise ValueError("rope_tables: pass cos and sin, or one complex tensor")
        cos, sin = cos.real, cos.imag
    while cos.dim() > 2 and cos.shape[0] == 1:
        cos, sin = cos[0], sin[0]
    if cos.dim() != 2 or cos.shape != sin.shape:
        raise ValueError("rope_tables: expected [tokens, pairs] or [tokens, head_dim] tables")
    return cos.float().contiguous(), sin.float().contiguous()


def _pair_tables(cos, sin, head_dim):
    if cos.shape[-1] == head_dim and head_dim > 1:
        cos, sin = cos[:, 0::2], sin[:, 0::2]
    if cos.shape[-1] != head_dim // 2:
        raise ValueError(f"rotary tables have {cos.shape[-1]} columns for head_dim {head_dim}")
    return cos.contiguous(), sin.contiguous()


def _as_bthd(x):
    """[T, H, D] or [B, T, H, D] -> a 4-D view."""
    if x.dim() == 3:
        return x.unsqueeze(0)
    if x.dim() != 4:
        raise ValueError("rotary input must be [tokens, heads, head_dim] or "
                         "[batch, tokens, heads, head_dim]")
    return x


class _RopeFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, cos, sin, inplace):
        x4 = _as_bthd(x)
        if inplace:
            out = x
            ctx.mark_dirty(x)
            rope_interleaved_apply(x4, cos, sin)
        else:
            out = x.clone(memory_format=torch.contiguous_format)
            rope_interleaved_apply(_as_bthd(out), cos, sin)
        ctx.save_for_backward(cos, sin)
        return out

    @staticmethod
    def backward(ctx, g):
        cos, sin = ctx.saved_tensors
        # the backward of a rotation is its transpose: the same kernel with
        # sin negated, on a private copy of the incoming gradient
        dx = g.clone(memory_format=torch.contiguous_format)
        rope_interleaved_apply(_as_bthd(dx), cos, sin, inverse=True)
        return dx, None, None, None


def apply_rotary_emb_interleaved(x, cos, sin=None, inplace=False):
    """Rotate interleaved pairs (x[2i], x[2i+1]) of x [B, T, H, D] or
    [T, H, D] by the token's angles.  Tables: see ``rope_tables``.  With
    ``inplace`` the input is overwritten (autograd records it)."""
    cos, sin = rope_tables(cos, sin)
    cos, sin = _pair_tables(cos, sin, x.shape[-1])
    if cos.shape[0] != x.shape[-3]:
        raise ValueError(f"rotary tables have {cos.shape[0]} tokens, input has {x.shape[-3]}")
    return _RopeFn.apply(x, cos, sin, bool(inplace))


# ---------------------------------------------------------------- RMSNorm -> RoPE

class _RMSNormRopeFn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x2, weight, cos, sin, head_dim, rows_per_token, eps, gemma):
        wk = _as_input_dtype(weight, x2)
        y, r = rmsnorm_rope_fwd(x2, wk, cos, sin, head_dim, rows_per_token, eps, gemma)
        ctx.save_for_backward(x2, wk, r, cos, sin)
        ctx.wdt = _dtype(weight)
        ctx.cfg = (head_dim, rows_per_token, gemma)
        return y

    @staticmethod
    def backward(ctx, dy):
        x2, weight, r, cos, sin = ctx.saved_tensors
        head_dim, rpt, gemma = ctx.cfg
        want_dw = weight is not None and ctx.needs_input_grad[1]
        dx, dw = rmsnorm_rope_bwd(_grad_rows(dy, x2), x2, weight, r, cos, sin, head_dim, rpt,
                                  gemma, want_dw=want_dw)
        return dx, _param_grad(dw, ctx.wdt), None, None, None, None, None, None


def rms_norm_rope(x, weight, cos, sin=None, eps=1e-6, gemma=False, per_head=False):
    """RoPE(RMSNorm(x)) in one pass each way, for x [B, T, H, D] or [T, H, D].

    per_head=False normalises each token's whole H*D vector (weight [H*D]);
    per_head=True normalises each head vector (weight [D], the q/k-norm of
    attention blocks).  Tables as for ``apply_rotary_emb_interleaved``; with
    a batch axis they are repeated per batch element for the kernel, which
    maps row i to table row i / rows_per_token."""
    x4 = _as_bthd(x)
    b, t, h, d = x4.shape
    cos, sin = rope_tables(cos, sin)
    cos, sin = _pair_tables(cos, sin, d)
    if cos.shape[0] != t:
        raise ValueError(f"rotary tables have {cos.shape[0]} tokens, input has {t}")
    if b > 1:
        cos, sin = cos.repeat(b, 1), sin.repeat(b, 1)
    if per_head:
        x2, rpt = x4.reshape(b * t * h, d), h
    else:
        x2, rpt = x4.reshape(b * t, h * d), 1
    y = _RMSNormRopeFn.apply(x2.contiguous(), weight, cos, sin, d, rpt, float(eps), bool(gemma))
    return y.view(x.shape)


# ---------------------------------------------------------------- modules

class FlashRMSNorm(nn.Module):
    """RMSNorm over the last axis on the fused kernel.  ``gemma``: the weight
    is stored as an offset from 1 (the module applies 1 + weight) and
    initialised to 0.  ``eps=None`` uses the machine epsilon of the input's
    dtype, as torch.nn.RMSNorm does."""

    def __init__(self, hidden_size, eps=1e-6, elementwise_affine=True, gemma=False, device=None,
                 dtype=None):
        super().__init__()
        self.hidden_size = int(hidden_size)
        self.eps = eps
        self.gemma = bool(gemma)
        if elementwise_affine:
            init = torch.zeros if gemma else torch.ones
            self.weight = nn.Parameter(init(self.hidden_size, device=device, dtype=dtype))
        else:
            self.register_parameter("weight", None)

    def forward(self, x):
        eps = torch.finfo(x.dtype).eps if self.eps is None else self.eps
        return rms_norm(x, self.weight, eps, self.gemma)

    def extra_repr(self):
        return f"{self.hidden_size}, eps={self.eps}, gemma={self.gemma}"


class FlashLayerNorm(nn.Module):
    """LayerNorm over the last axis on the fused kernel (biased variance,
    eps inside the root, optional weight and bias), like torch.nn.LayerNorm
    with a one-axis normalized_shape."""

    _gelu = False

    def __init__(self, normalized_shape, eps=1e-5, elementwise_affine=True, bias=True,
                 device=None, dtype=None):
        super().__init__()
        if isinstance(normalized_shape, (tuple, list, torch.Size)):
            if len(normalized_shape) != 1:
                raise ValueError("FlashLayerNorm normalises the last axis only")
            normalized_shape = normalized_shape[0]
        self.normalized_shape = (int(normalized_shape),)
        self.eps = float(eps)
        if elementwise_affine:
            self.weight = nn.Parameter(torch.ones(self.normalized_shape, device=device, dtype=dtype))
            if bias:
                self.bias = nn.Parameter(torch.zeros(self.normalized_shape, device=device,
                                                     dtype=dtype))
            else:
                self.register_parameter("bias", None)
        else:
            self.register_parameter("weight", None)
            self.register_parameter("bias", None)

    def forward(self, x):
        fn = layer_norm_gelu if self._gelu else layer_norm
        return fn(x, self.weight, self.bias, self.eps)

    def extra_repr(self):
        return f"{self.normalized_shape}, eps={self.eps}"


class FlashLayerNormGelu(FlashLayerNorm):
    """gelu_tanh(LayerNorm(x)) in one kernel per direction (the fused
    LayerNorm + GeLU of "LLM层的优化算子", 编写定制融合算子)."""

    _gelu = True


# ---------------------------------------------------------------- patches

def _rms_eps(mod):
    for attr in ("eps", "variance_epsilon", "epsilon"):
        v = getattr(mod, attr, None)
        if v is None and attr == "eps" and isinstance(mod, getattr(nn, "RMSNorm", ())):
            return None  # torch.nn.RMSNorm: machine epsilon of the input dtype
        if isinstance(v, (int, float)):
            return float(v)
    raise ValueError(f"{type(mod).__name__}: no eps attribute")


def _is_rmsnorm(mod):
    if isinstance(mod, getattr(nn, "RMSNorm", ())):
        shape = tuple(mod.normalized_shape)
        return len(shape) == 1
    name = type(mod).__name__
    w = getattr(mod, "weight", None)
    return (name.endswith("RMSNorm") and not isinstance(mod, FlashRMSNorm)
            and (w is None or (isinstance(w, nn.Parameter) and w.dim() == 1)))


def _flash_rms_from(mod):
    w = getattr(mod, "weight", None)
    if isinstance(mod, getattr(nn, "RMSNorm", ())):
        hidden = mod.normalized_shape[0]
    elif w is not None:
        hidden = w.shape[0]
    else:
        hidden = int(getattr(mod, "hidden_size", getattr(mod, "dim", 0)))
    gemma = "Gemma" in type(mod).__name__
    new = FlashRMSNorm(hidden, _rms_eps(mod), elementwise_affine=False, gemma=gemma)
    new.weight = w  # the same Parameter object: optimiser state and tying stay intact
    return new


def _flash_ln_from(mod):
    new = FlashLayerNorm(mod.normalized_shape, mod.eps, elementwise_affine=False)
    new.weight, new.bias = mod.weight, mod.bias
    return new


def _swap(model, pick, build):
    count = 0
    for parent in list(model.modules()):
        for name, child in list(parent.named_children()):
            if pick(child):
                setattr(parent, name, build(child))
                count += 1
    return count


def replace_all_norms_with_flash_norms(model: nn.Module, rmsnorm=True, layernorm=True) -> int:
    """Swap every one-axis torch.nn.LayerNorm and every RMSNorm module
    (torch.nn.RMSNorm, or a class whose name ends in "RMSNorm" with a 1-D
    weight and an eps / variance_epsilon attribute; "Gemma" in the class
    name selects the 1 + w form) for the fused-kernel modules, in place.
    The new modules hold the same Parameter objects.  Returns the number of
    modules replaced."""
    n = 0
    if layernorm:
        n += _swap(model, lambda m: isinstance(m, nn.LayerNorm) and len(m.normalized_shape) == 1,
                   _flash_ln_from)
    if rmsnorm:
        n += _swap(model, _is_rmsnorm, _flash_rms_from)
    return n


def replace_rmsnorm_with_fp32(model: nn.Module) -> int:
    """Swap only the RMSNorm modules (see replace_all_norms_with_flash_norms).
    The fused kernels accumulate in fp32 and round the output once, whatever
    the storage dtype, which is what an fp32-precision RMSNorm is for."""
    return replace_all_norms_with_flash_norms(model, rmsnorm=True, layernorm=False)


def replace_rope_with_flash_rope(namespace, name="apply_rotary_emb", adapter=None):
    """Replace the function ``namespace.name`` (a module or object attribute)
    by the interleaved-RoPE kernel, so every caller that looks it up there
    takes the fused path.  ``adapter(x, *args, **kwargs) -> (x, cos, sin)``
    maps the original signature onto ours; by default the call is forwarded
    as apply_rotary_emb_interleaved(x, cos, sin).  Returns the original
    function (setattr it back to undo)."""
    original = getattr(namespace, name)

    def flash_rope(x, *args, **kwargs):
        if adapter is not None:
            x, cos, sin = adapter(x, *args, **kwargs)
            return apply_rotary_emb_interleaved(x, cos, sin)
        return apply_rotary_emb_interleaved(x, *args, **kwargs)

    flash_rope.__name__ = f"flash_{name}"
    flash_rope.__wrapped__ = original
    setattr(namespace, name, flash_rope)
    return original
