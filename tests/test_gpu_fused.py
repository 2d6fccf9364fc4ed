"""GPU parity of the fused RMSNorm + RoPE pair against the oracle's fp64
composition (no intermediate rounding on either side of the comparison: the
fused kernels round once, so the plain 1-ulp bound applies)."""
import numpy as np
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, grad_scale, out_kind, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[case] {msg}", flush=True)


def g(t):
    return None if t is None else t.to(DEV)


def check_fused(tag, x, w, dout, ang, head_dim, rows_per_token, gemma=False, eps=1e-6,
                layout="packed"):
    rows, n = x.shape
    tokens = ang.shape[0]
    say(f"{tag}: fused rmsnorm+rope {rows}x{n} head_dim={head_dim} rows/token={rows_per_token} "
        f"{x.dtype} gemma={gemma} {layout}")
    ct = torch.from_numpy(np.cos(ang)).float().to(DEV)
    st = torch.from_numpy(np.sin(ang)).float().to(DEV)
    if layout == "unaligned":
        buf = torch.empty(rows * n + 1, dtype=x.dtype, device=DEV)
        xg = buf[1:].view(rows, n)
        xg.copy_(g(x))
    else:
        xg = g(x)
    y, r = nr.rmsnorm_rope_fwd(xg, g(w), ct, st, head_dim, rows_per_token, eps, gemma)
    dx, dw = nr.rmsnorm_rope_bwd(g(dout), xg, g(w), r, ct, st, head_dim, rows_per_token, gemma)
    torch.cuda.synchronize()
    ry, rr = oracle.rmsnorm_rope_fwd(x, w, ang, head_dim, rows_per_token, eps, gemma)
    rdx, rdw = oracle.rmsnorm_rope_bwd(dout, x, w, ang, head_dim, rows_per_token, eps, gemma)
    k = out_kind(x.dtype)
    check(f"{tag} y", y, ry, k)
    check(f"{tag} inv_rms", r, rr, "stat", s=0.0)
    dy64 = oracle.rope_apply(dout.reshape(1, rows, n // head_dim, head_dim),
                             ang[np.arange(rows) // rows_per_token], inverse=True).reshape(rows, n)
    check(f"{tag} dx", dx, rdx, k, s=grad_scale(rr, dy64, w, gemma))
    if w is not None:
        check(f"{tag} dw", dw, rdw, "col")
    # the table built by the library gives the same result within the bound
    return ct, st


# (rows, heads per row, head_dim, rows_per_token, dtype, gemma, layout)
CASES = [
    (64, 4, 64, 1, torch.float32, False, "packed"),
    (99, 40, 128, 1, torch.bfloat16, False, "packed"),
    (132, 1, 64, 4, torch.bfloat16, True, "packed"),      # each head normalised on its own
    (50, 3, 6, 1, torch.bfloat16, False, "packed"),       # head_dim 6: element-wise path
    (40, 2, 32, 2, torch.float32, True, "packed"),
    (33, 8, 128, 1, torch.bfloat16, False, "unaligned"),
    (77, 40, 128, 1, torch.float16, False, "packed"),
    (48, 2, 64, 2, torch.float16, True, "packed"),
    # two chunks per lane in the backward: one set of angles per row where the
    # lane stride is a multiple of the head size, one per chunk where not (96)
    (37, 96, 128, 1, torch.bfloat16, False, "packed"),    # 12288 wide, 12 waves
    (29, 120, 128, 1, torch.float16, True, "packed"),     # 15360 wide, 15 waves
    (31, 48, 128, 1, torch.float32, False, "packed"),     # 6144 fp32, 12 waves
    (23, 100, 96, 1, torch.bfloat16, False, "packed"),    # 9600 wide: 5120 % 96 != 0
    (21, 160, 128, 1, torch.bfloat16, False, "packed"),   # 20480 wide: two-pass backward
    (9, 170, 102, 1, torch.float32, True, "packed"),      # 17340 wide, element-wise tables
    # per-head rows (a q/k norm): the packed kernels, on enough rows for the
    # backward's full workgroup count, and the wave-per-row kernels unaligned
    (90001, 1, 128, 40, torch.bfloat16, False, "packed"),
    (20000, 1, 64, 8, torch.float16, True, "packed"),
    (3001, 1, 128, 8, torch.bfloat16, False, "unaligned"),
]


@pytest.mark.parametrize("rows,heads,d,rpt,dtype,gemma,layout", CASES)
def test_fused_cases(rows, heads, d, rpt, dtype, gemma, layout):
    n = heads * d
    seed = 7000 + rows + n
    x = workloads.normal((rows, n), seed, dtype)
    w = workloads.normal((n,), seed + 1, dtype, mean=0.0 if gemma else 1.0, std=0.1)
    dout = workloads.normal((rows, n), seed + 2, dtype)
    ang = oracle.rope_angles_1d(-(-rows // rpt), d, 5, 10000.0)
    check_fused(f"fused {rows}x{heads}x{d}", x, w, dout, ang, d, rpt, gemma, layout=layout)


def test_fused_in_place_and_library_table():
    rows, heads, d = 70, 4, 64
    n = heads * d
    x = workloads.normal((rows, n), 7101, torch.bfloat16)
    w = workloads.normal((n,), 7102, torch.bfloat16, mean=1.0, std=0.1)
    dout = workloads.normal((rows, n), 7103, torch.bfloat16)
    ang = oracle.rope_angles_1d(rows, d, 0, 10000.0)
    ry, rr = oracle.rmsnorm_rope_fwd(x, w, ang, d)
    rdx, rdw = oracle.rmsnorm_rope_bwd(dout, x, w, ang, d)
    say("fused in place (y == x, dx == dout) with library-built tables")
    ct, st = nr.rope_table_1d(rows, d, 0, 10000.0)
    xg, gg = g(x), g(dout)
    _, r = nr.rmsnorm_rope_fwd(xg.clone(), g(w), ct, st, d)
    nr.rmsnorm_rope_bwd(gg, xg, g(w), r, ct, st, d, dx=gg)
    nr.rmsnorm_rope_fwd(xg, g(w), ct, st, d, y=xg)
    torch.cuda.synchronize()
    check("in-place y", xg, ry, "bf16")
    dy64 = oracle.rope_apply(dout.reshape(1, rows, heads, d), ang, inverse=True).reshape(rows, n)
    check("in-place dx", gg, rdx, "bf16", s=grad_scale(rr, dy64, w))


def test_fused_longseq():
    """Every row of y, inv_rms and dx of the fused chain at 65536 x 5120, and
    the full dw, the oracle taken in blocks of 4096 rows."""
    inp = workloads.norm_inputs("longseq_65536x5120")
    x, w, dout, eps = inp["x"], inp["w"], inp["dy"], inp["eps"]
    m, n = x.shape
    d = 128
    say("fused longseq_65536x5120: rmsnorm+rope fwd and bwd, every row + full dw")
    ct, st = nr.rope_table_1d(m, d, 0, 10000.0)
    y, r = nr.rmsnorm_rope_fwd(g(x), g(w), ct, st, d, 1, eps)
    dx, dw = nr.rmsnorm_rope_bwd(g(dout), g(x), g(w), r, ct, st, d)
    torch.cuda.synchronize()
    y, r, dx = y.cpu(), r.cpu(), dx.cpu()
    ang = oracle.rope_angles_1d(m, d, 0, 10000.0)
    rdw = np.zeros(n)
    for b0 in range(0, m, 4096):
        sl = slice(b0, b0 + 4096)
        xs, ds, a = x[sl], dout[sl], ang[sl]
        ry, rr = oracle.rmsnorm_rope_fwd(xs, w, a, d, 1, eps)
        rdx, bdw = oracle.rmsnorm_rope_bwd(ds, xs, w, a, d, 1, eps)
        rdw += bdw
        check(f"fused longseq y rows {b0}..", y[sl], ry, "bf16")
        check(f"fused longseq inv_rms rows {b0}..", r[sl], rr, "stat", s=0.0)
        dy64 = oracle.rope_apply(ds.reshape(1, xs.shape[0], n // d, d), a, inverse=True)
        check(f"fused longseq dx rows {b0}..", dx[sl], rdx, "bf16",
              s=grad_scale(rr, dy64.reshape(xs.shape[0], n), w))
    # dw over every row: the blocks' fp64 column sums added in fp64
    check("fused longseq dw", dw, rdw, "col")


# ---------------------------------------------------------------- LayerNorm + GeLU

def check_ln_gelu(tag, x, gm, bt, dout, eps=1e-5, layout="packed"):
    rows, n = x.shape
    say(f"{tag}: fused layernorm+gelu {rows}x{n} {x.dtype} gamma={gm is not None} "
        f"beta={bt is not None} {layout}")
    if layout == "unaligned":
        buf = torch.empty(rows * n + 1, dtype=x.dtype, device=DEV)
        xg = buf[1:].view(rows, n)
        xg.copy_(g(x))
    else:
        xg = g(x)
    y, mu, rs = nr.layernorm_gelu_fwd(xg, g(gm), g(bt), eps)
    dx, dg, db = nr.layernorm_gelu_bwd(g(dout), xg, g(gm), g(bt), mu, rs)
    torch.cuda.synchronize()
    ry, rmu, rrs = oracle.layernorm_gelu_fwd(x, gm, bt, eps)
    rdx, rdg, rdb = oracle.layernorm_gelu_bwd(dout, x, gm, bt, eps)
    k = out_kind(x.dtype)
    x64 = to64(x)
    check(f"{tag} y", y, ry, k)
    check(f"{tag} mean", mu, rmu, "stat", s=np.sqrt(np.mean(x64 * x64, axis=1)))
    check(f"{tag} rstd", rs, rrs, "stat", s=0.0)
    # row scale of dx: the terms r * dout * gamma (|gelu'| stays below 1.13)
    check(f"{tag} dx", dx, rdx, k, s=1.13 * grad_scale(rrs, dout, gm))
    check(f"{tag} dgamma", dg, rdg, "col")
    check(f"{tag} dbeta", db, rdb, "col")


def test_ln_gelu_full_size():
    inp = workloads.norm_inputs("ln_affine_15360x5120")
    check_ln_gelu("ln_gelu_15360x5120", inp["x"], inp["w"], inp["b"], inp["dy"], inp["eps"])


@pytest.mark.parametrize("rows,n,dtype,affine,layout", [
    (1, 1, torch.float32, True, "packed"), (3, 7, torch.bfloat16, True, "packed"),
    (257, 64, torch.float32, True, "packed"), (33, 1000, torch.bfloat16, False, "packed"),
    (17, 5128, torch.bfloat16, True, "packed"), (9, 8191, torch.bfloat16, True, "packed"),
    (40, 520, torch.bfloat16, True, "unaligned"), (3, 32768, torch.float32, True, "packed"),
    (45, 5120, torch.float16, True, "packed"), (6, 1003, torch.float16, True, "packed"),
    (7, 20480, torch.bfloat16, True, "packed"), (5, 17003, torch.bfloat16, True, "unaligned"),
    # 16-bit rows of 2560 and 5120: the backward's 10-elements-a-lane layout
    (300, 2560, torch.bfloat16, True, "packed"), (513, 5120, torch.bfloat16, False, "packed"),
    (77, 2560, torch.float16, True, "packed"), (1, 5120, torch.bfloat16, True, "packed"),
    (31, 2560, torch.bfloat16, True, "unaligned"), (8200, 2560, torch.bfloat16, True, "packed"),
])
def test_ln_gelu_edges(rows, n, dtype, affine, layout):
    seed = 8000 + rows * 3 + n
    x = workloads.normal((rows, n), seed, dtype, mean=0.5, std=2.0)
    gm = workloads.normal((n,), seed + 1, dtype, mean=1.0, std=0.1) if affine else None
    bt = workloads.normal((n,), seed + 2, dtype, std=0.5) if affine else None
    dout = workloads.normal((rows, n), seed + 3, dtype)
    check_ln_gelu(f"ln+gelu edge {rows}x{n}", x, gm, bt, dout, layout=layout)


@pytest.mark.parametrize("which,n", [("gamma", 5120), ("beta", 5120), ("gamma", 2560), ("beta", 2560)])
def test_ln_gelu_one_affine_parameter(which, n):
    # gamma without beta and beta without gamma, on the widths whose backward
    # takes 10 elements a lane (a missing gamma is 1, a missing beta 0)
    rows = 129
    seed = 8800 + n + (which == "beta")
    x = workloads.normal((rows, n), seed, torch.bfloat16, mean=0.5, std=2.0)
    gm = workloads.normal((n,), seed + 1, torch.bfloat16, mean=1.0, std=0.1) if which == "gamma" else None
    bt = workloads.normal((n,), seed + 2, torch.bfloat16, std=0.5) if which == "beta" else None
    dout = workloads.normal((rows, n), seed + 3, torch.bfloat16)
    check_ln_gelu(f"ln+gelu {which} only {rows}x{n}", x, gm, bt, dout)
