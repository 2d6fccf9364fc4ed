"""Seeded synthetic inputs for the norm and RoPE operators.

This module only draws numbers and rounds them to the storage dtype.  It holds
none of the operators' arithmetic: no normalisation, no rotation, no RoPE
angle or frequency.  Both the HIP path (tests, bench) and the fp64 oracle are
fed from here, so the two sides see identical input bytes.

Recipe (one entry per workload below):
  * generator: numpy PCG64 seeded with ``1000 + index``; independent
    sub-streams come from ``SeedSequence(seed).spawn(8)`` in the fixed order
    x, weight/gamma, beta, dy/dout, outlier rows, q, k, spare;
  * values are drawn as float32 standard normals, scaled/shifted in float32,
    then rounded once to the storage dtype (bf16 by round-to-nearest-even);
  * the Helios video model whose layers these shapes come from (hidden 5120,
    40 heads of 128, tens of thousands of tokens) is not available here, so
    these draws stand in for its activations.
"""
from __future__ import annotations

import numpy as np
import torch

# sub-stream slots, fixed order
_X, _W, _B, _DY, _OUT, _Q, _K, _SPARE = range(8)

WORKLOADS = {
    # fp32 parity case small enough for pure-Python checks
    "tiny_f32": dict(
        index=1, dtype=torch.float32,
        norm=dict(kind="rms", rows=64, n=256, x=(0.0, 1.0), w=("1+", 0.1),
                  eps=1e-6, gemma=False),
        rope=dict(shape=(1, 64, 4, 64), tensors=("q",),
                  table=dict(kind="1d", pos0=0, theta=10000.0)),
    ),
    # RMSNorm fwd+bwd with the Gemma (1 + w) weight offset
    "rms_gemma_3840x5120": dict(
        index=2, dtype=torch.bfloat16,
        norm=dict(kind="rms", rows=3840, n=5120, x=(0.0, 1.0), w=("", 0.1),
                  eps=1e-6, gemma=True),
    ),
    # affine LayerNorm fwd+bwd
    "ln_affine_15360x5120": dict(
        index=3, dtype=torch.bfloat16,
        norm=dict(kind="ln", rows=15360, n=5120, x=(0.5, 2.0), w=("1+", 0.1),
                  b=0.1, eps=1e-5),
    ),
    # RoPE on q and k with a 3-D (frames x height x width) position grid
    "rope3d_15360x40x128": dict(
        index=4, dtype=torch.bfloat16,
        rope=dict(shape=(1, 15360, 40, 128), tensors=("q", "k"),
                  table=dict(kind="3d", grid=(16, 24, 40), pairs=(22, 21, 21),
                             theta=10000.0)),
    ),
    # long-sequence chain: RMSNorm fwd -> RoPE, RoPE inverse -> RMSNorm bwd
    "longseq_65536x5120": dict(
        index=5, dtype=torch.bfloat16,
        norm=dict(kind="rms", rows=65536, n=5120, x=(0.0, 1.0), w=("1+", 0.1),
                  eps=1e-6, gemma=False, outlier_frac=0.01, outlier_scale=100.0),
        rope=dict(shape=(1, 65536, 40, 128), tensors=(),
                  table=dict(kind="1d", pos0=0, theta=10000.0)),
    ),
}


def _streams(index: int):
    ss = np.random.SeedSequence(1000 + index)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(8)]


def _to(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 numpy array -> CPU tensor of ``dtype`` (one RNE rounding)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if dtype == torch.float32 else t.to(dtype)


def normal(shape, seed: int, dtype=torch.float32, mean=0.0, std=1.0,
           slot: int = _SPARE) -> torch.Tensor:
    """Generic seeded N(mean, std^2) draw for edge-case tests."""
    rng = _streams(seed - 1000)[slot]
    z = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        z *= np.float32(std)
    if mean != 0.0:
        z += np.float32(mean)
    return _to(z, dtype)


def normal_device(shape, seed: int, dtype=torch.bfloat16, device="cuda", mean=0.0, std=1.0,
                  block_rows: int = 1 << 18) -> torch.Tensor:
    """Seeded N(mean, std^2) draw made on the device, for tensors too large to
    draw on the host (several GiB): torch's device generator seeded with
    ``seed``, drawn in float32 blocks of rows, each rounded once to ``dtype``.
    The same seed and shape give the same values on the same device type."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], block_rows):
        r1 = min(shape[0], r0 + block_rows)
        z = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            z.mul_(std)
        if mean != 0.0:
            z.add_(mean)
        flat[r0:r1] = z.to(dtype)
    return out


def norm_inputs(name: str) -> dict:
    """x, weight, bias, dy for a workload's norm step (CPU tensors)."""
    wl = WORKLOADS[name]
    spec = wl["norm"]
    dt = wl["dtype"]
    st = _streams(wl["index"])
    m, n = spec["rows"], spec["n"]
    mean, std = spec["x"]
    x = st[_X].standard_normal((m, n), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    if spec.get("outlier_frac"):
        k = int(round(spec["outlier_frac"] * m))
        rows = np.sort(st[_OUT].permutation(m)[:k])
        x[rows] *= np.float32(spec["outlier_scale"])
    else:
        rows = np.zeros(0, dtype=np.int64)
    wkind, wstd = spec["w"]
    w = st[_W].standard_normal(n, dtype=np.float32) * np.float32(wstd)
    if wkind == "1+":
        w += np.float32(1.0)
    b = None
    if "b" in spec:
        b = st[_B].standard_normal(n, dtype=np.float32) * np.float32(spec["b"])
    dy = st[_DY].standard_normal((m, n), dtype=np.float32)
    out = dict(kind=spec["kind"], x=_to(x, dt), w=_to(w, dt),
               b=None if b is None else _to(b, dt), dy=_to(dy, dt),
               eps=spec["eps"], gemma=spec.get("gemma", False),
               outlier_rows=torch.from_numpy(rows))
    return out


def rope_inputs(name: str) -> dict:
    """Tensors to rotate (CPU, [B, T, H, D]) and the table's parameters."""
    wl = WORKLOADS[name]
    spec = wl["rope"]
    dt = wl["dtype"]
    st = _streams(wl["index"])
    shape = spec["shape"]
    out = dict(shape=shape, table=dict(spec["table"]))
    for nm in spec["tensors"]:
        slot = _Q if nm == "q" else _K
        out[nm] = _to(st[slot].standard_normal(shape, dtype=np.float32), dt)
    return out
