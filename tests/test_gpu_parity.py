"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every test feeds both sides the same seeded input bytes; the oracle never
sees a GPU output (chained checks compare against the oracle's own fp64
chain, with a bound derived from the one extra rounding in between).  The
bounds are written out in tests/tolerance.py.  The full-size workloads run
in the launch configuration the benchmark times (the library's automatic
choice).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
import workloads
from tolerance import check, grad_scale, out_kind, to64, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(msg):
    print(f"[case] {msg}", flush=True)


def g(t):
    return None if t is None else t.to(DEV)


def ulp32(c):
    a = np.abs(c)
    _, e = np.frexp(a)
    return np.where(a > 0, np.ldexp(1.0, e - 24), 2.0 ** -149)


def check_table(name, cos_t, sin_t, angle):
    """fp32 tables against cos/sin of the oracle's fp64 angles: one fp32 ulp,
    plus what the two sides' double-precision angles (each within a few
    2^-53 relative of the true angle) can differ by: 4e-15 |angle|."""
    c, s = to64(cos_t), to64(sin_t)
    rc, rs = np.cos(angle), np.sin(angle)
    slack = 4e-15 * np.abs(angle)
    for nm, o, r in (("cos", c, rc), ("sin", s, rs)):
        err = np.abs(o - r)
        tol = ulp32(r) + slack
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        assert np.all(err <= tol), (f"{name} {nm}: worst at {i}: angle={angle[i]!r} gpu={o[i]!r} "
                                    f"oracle={r[i]!r} err={err[i]:.3e} bound={tol[i]:.3e}")


# ---------------------------------------------------------------- RMSNorm

def run_rms(x, w, dy, eps, gemma, want_dw=True):
    y, r = nr.rmsnorm_fwd(g(x), g(w), eps=eps, gemma_offset=gemma)
    dx, dw = nr.rmsnorm_bwd(g(dy), g(x), g(w), r, gemma_offset=gemma, want_dw=want_dw)
    torch.cuda.synchronize()
    return y, r, dx, dw


def check_rms_full(tag, x, w, dy, eps, gemma):
    say(f"{tag}: rmsnorm fwd+bwd {tuple(x.shape)} {x.dtype} gemma={gemma} w={'yes' if w is not None else 'none'}")
    y, r, dx, dw = run_rms(x, w, dy, eps, gemma, want_dw=w is not None)
    ry, rr = oracle.rmsnorm_fwd(x, w, eps, gemma)
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, eps, gemma, want_dw=w is not None)
    k = out_kind(x.dtype)
    n = x.shape[-1]
    check(f"{tag} y", y.reshape(-1, n), ry, k)
    check(f"{tag} inv_rms", r.reshape(-1), rr, "stat", s=0.0)
    check(f"{tag} dx", dx.reshape(-1, n), rdx, k, s=grad_scale(rr, dy, w, gemma))
    if w is not None:
        check(f"{tag} dw", dw, rdw, "col")


def test_tiny_f32_rmsnorm():
    inp = workloads.norm_inputs("tiny_f32")
    check_rms_full("tiny_f32", inp["x"], inp["w"], inp["dy"], inp["eps"], inp["gemma"])


def test_rms_gemma_3840x5120():
    inp = workloads.norm_inputs("rms_gemma_3840x5120")
    check_rms_full("rms_gemma_3840x5120", inp["x"], inp["w"], inp["dy"], inp["eps"], True)


# ---------------------------------------------------------------- LayerNorm

def check_ln_full(tag, x, gm, bt, dy, eps):
    say(f"{tag}: layernorm fwd+bwd {tuple(x.shape)} {x.dtype} gamma={gm is not None} beta={bt is not None}")
    y, mu, rs = nr.layernorm_fwd(g(x), g(gm), g(bt), eps=eps)
    dx, dg, db = nr.layernorm_bwd(g(dy), g(x), g(gm), mu, rs)
    torch.cuda.synchronize()
    ry, rmu, rrs = oracle.layernorm_fwd(x, gm, bt, eps)
    rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, gm, eps)
    k = out_kind(x.dtype)
    n = x.shape[-1]
    x64 = to64(x).reshape(-1, n)
    check(f"{tag} y", y.reshape(-1, n), ry, k)
    check(f"{tag} mean", mu.reshape(-1), rmu, "stat", s=np.sqrt(np.mean(x64 * x64, axis=1)))
    check(f"{tag} rstd", rs.reshape(-1), rrs, "stat", s=0.0)
    check(f"{tag} dx", dx.reshape(-1, n), rdx, k, s=grad_scale(rrs, dy, gm))
    check(f"{tag} dgamma", dg, rdg, "col")
    check(f"{tag} dbeta", db, rdb, "col")


def test_ln_affine_15360x5120():
    inp = workloads.norm_inputs("ln_affine_15360x5120")
    check_ln_full("ln_affine_15360x5120", inp["x"], inp["w"], inp["b"], inp["dy"], inp["eps"])


# ---------------------------------------------------------------- RoPE

def gpu_table(spec, tokens, head_dim):
    if spec["kind"] == "1d":
        return nr.rope_table_1d(tokens, head_dim, spec.get("pos0", 0), spec["theta"])
    return nr.rope_table_3d(spec["grid"], spec["pairs"], spec["theta"])


def check_rope_full(tag, x, spec):
    b, t, h, d = x.shape
    say(f"{tag}: rope table + fwd/inverse {tuple(x.shape)} {x.dtype} table={spec['kind']}")
    ct, st = gpu_table(spec, t, d)
    ang = oracle.rope_angles(spec, t, d)
    torch.cuda.synchronize()
    check_table(tag, ct, st, ang)
    k = out_kind(x.dtype)
    for inv in (False, True):
        xg = g(x).clone()
        nr.rope_interleaved_apply(xg, ct, st, inverse=inv)
        torch.cuda.synchronize()
        ref = oracle.rope_apply(x, ang, inv)
        check(f"{tag} {'inverse' if inv else 'forward'}", xg.reshape(-1, d), ref.reshape(-1, d), k)
    # forward then inverse returns the input; the bound allows the rounding of
    # the intermediate (half an ulp of each element of the rotated pair)
    xg = g(x).clone()
    nr.rope_interleaved_apply(xg, ct, st)
    nr.rope_interleaved_apply(xg, ct, st, inverse=True)
    torch.cuda.synchronize()
    x64 = to64(x).reshape(-1, 2)
    pair = np.repeat(np.sqrt((x64 ** 2).sum(axis=1)), 2)
    extra = 0.0 if x.dtype == torch.float32 else (2 ** -8) * math.sqrt(2) * 1.01 * pair
    check(f"{tag} round trip", xg.reshape(-1), to64(x).reshape(-1), k, s=0.0,
          extra=extra if x.dtype == torch.bfloat16 else 1e-6 * pair)


def test_tiny_f32_rope():
    inp = workloads.rope_inputs("tiny_f32")
    check_rope_full("tiny_f32", inp["q"], inp["table"])


@pytest.mark.parametrize("which", ["q", "k"])
def test_rope3d_15360x40x128(which):
    inp = workloads.rope_inputs("rope3d_15360x40x128")
    check_rope_full(f"rope3d_15360x40x128 {which}", inp[which], inp["table"])


# ---------------------------------------------------------------- long sequence

@pytest.fixture(scope="module")
def longseq():
    inp = workloads.norm_inputs("longseq_65536x5120")
    spec = workloads.WORKLOADS["longseq_65536x5120"]["rope"]
    return inp, spec


def row_blocks(m, bs=4096):
    """Every row, in host-side blocks (bounded fp64 memory)."""
    for b0 in range(0, m, bs):
        yield b0, min(m, b0 + bs)


def test_longseq_rmsnorm(longseq):
    """Every row of y, inv_rms and dx, and the full dw, at the benchmark's
    shape and launch configuration (outlier rows included)."""
    inp, _ = longseq
    x, w, dy, eps = inp["x"], inp["w"], inp["dy"], inp["eps"]
    say("longseq_65536x5120: rmsnorm fwd+bwd, every row + full dw")
    y, r, dx, dw = run_rms(x, w, dy, eps, False)
    y, r, dx = y.cpu(), r.cpu(), dx.cpu()
    for b0, b1 in row_blocks(65536):
        ry, rr = oracle.rmsnorm_fwd(x[b0:b1], w, eps)
        rdx, _ = oracle.rmsnorm_bwd(dy[b0:b1], x[b0:b1], w, eps, want_dw=False)
        check(f"longseq y rows {b0}..", y[b0:b1], ry, "bf16")
        check(f"longseq inv_rms rows {b0}..", r[b0:b1], rr, "stat", s=0.0)
        check(f"longseq dx rows {b0}..", dx[b0:b1], rdx, "bf16", s=grad_scale(rr, dy[b0:b1], w))
    _, rdw = oracle.rmsnorm_bwd(dy, x, w, eps, want_dx=False)
    check("longseq dw", dw, rdw, "col")


def test_longseq_layernorm(longseq):
    """LayerNorm fwd+bwd at the benchmark's long-sequence shape (x and dout of
    the long sequence, gamma and beta of the affine workload, eps 1e-5):
    every row of y, mean, rstd and dx, and the full dgamma and dbeta."""
    inp, _ = longseq
    lnp = workloads.norm_inputs("ln_affine_15360x5120")
    x, dy, gm, bt, eps = inp["x"], inp["dy"], lnp["w"], lnp["b"], 1e-5
    say("longseq_65536x5120: layernorm fwd+bwd, every row + full dgamma, dbeta")
    y, mu, rs = nr.layernorm_fwd(g(x), g(gm), g(bt), eps=eps)
    dx, dg, db = nr.layernorm_bwd(g(dy), g(x), g(gm), mu, rs)
    torch.cuda.synchronize()
    y, mu, rs, dx = y.cpu(), mu.cpu(), rs.cpu(), dx.cpu()
    for b0, b1 in row_blocks(65536):
        ry, rmu, rrs = oracle.layernorm_fwd(x[b0:b1], gm, bt, eps)
        rdx, _, _ = oracle.layernorm_bwd(dy[b0:b1], x[b0:b1], gm, eps, want_dw=False)
        x64 = to64(x[b0:b1])
        check(f"longseq ln y rows {b0}..", y[b0:b1], ry, "bf16")
        check(f"longseq ln mean rows {b0}..", mu[b0:b1], rmu, "stat",
              s=np.sqrt(np.mean(x64 * x64, axis=1)))
        check(f"longseq ln rstd rows {b0}..", rs[b0:b1], rrs, "stat", s=0.0)
        check(f"longseq ln dx rows {b0}..", dx[b0:b1], rdx, "bf16", s=grad_scale(rrs, dy[b0:b1], gm))
    _, rdg, rdb = oracle.layernorm_bwd(dy, x, gm, eps, want_dx=False)
    check("longseq dgamma", dg, rdg, "col")
    check("longseq dbeta", db, rdb, "col")


def test_longseq_rope(longseq):
    inp, spec = longseq
    d, h = 128, 40
    ang = oracle.rope_angles(spec["table"], 65536, d)
    say("longseq_65536x5120: rope table 1-D 65536 tokens")
    ct, st = gpu_table(spec["table"], 65536, d)
    torch.cuda.synchronize()
    check_table("longseq", ct, st, ang)
    for name, src, inv in (("x forward", inp["x"], False), ("dout inverse", inp["dy"], True)):
        say(f"longseq_65536x5120: rope {name}, every token")
        xg = g(src).view(1, 65536, h, d).clone()
        nr.rope_interleaved_apply(xg, ct, st, inverse=inv)
        torch.cuda.synchronize()
        xg = xg.cpu()
        for b0, b1 in row_blocks(65536, 8192):
            ref = oracle.rope_apply(src[b0:b1].view(1, b1 - b0, h, d), ang[b0:b1], inv)
            check(f"longseq rope {name} tokens {b0}..", xg[0, b0:b1].reshape(-1, d), ref.reshape(-1, d),
                  "bf16")


def test_longseq_chain(longseq):
    """norm -> RoPE forward, and RoPE inverse -> norm backward, against the
    oracle's fp64 chain, every row.  The GPU rounds the intermediate to bf16
    once; the bound adds what that rounding can move the final value by."""
    inp, spec = longseq
    x, w, dout, eps = inp["x"], inp["w"], inp["dy"], inp["eps"]
    d, h = 128, 40
    angs = oracle.rope_angles(spec["table"], 65536, d)
    say("longseq_65536x5120: chain rmsnorm -> rope")
    ct, st = gpu_table(spec["table"], 65536, d)
    y, r = nr.rmsnorm_fwd(g(x), g(w), eps=eps)
    nr.rope_interleaved_apply(y.view(1, 65536, h, d), ct, st)
    say("longseq_65536x5120: chain rope inverse -> rmsnorm bwd")
    dyg = g(dout).view(1, 65536, h, d).clone()
    nr.rope_interleaved_apply(dyg, ct, st, inverse=True)
    dx, _ = nr.rmsnorm_bwd(dyg.view(65536, -1), g(x), g(w), r, want_dw=False)
    torch.cuda.synchronize()
    y, dx = y.cpu(), dx.cpu()
    for b0, b1 in row_blocks(65536):
        nb, ang = b1 - b0, angs[b0:b1]
        ry, _ = oracle.rmsnorm_fwd(x[b0:b1], w, eps)
        ref = oracle.rope_apply(torch.from_numpy(ry).view(1, nb, h, d), ang)
        pair = np.abs(ry).reshape(-1, 2).sum(axis=1)
        extra = (2 ** -8) * 1.01 * np.repeat(pair, 2).reshape(nb, -1)
        check(f"chain fwd rows {b0}..", y[b0:b1], ref.reshape(nb, -1), "bf16", extra=extra)
        dy64 = oracle.rope_apply(dout[b0:b1].view(1, nb, h, d), ang, inverse=True).reshape(nb, -1)
        xs = x[b0:b1].double()
        rdx, _ = oracle.rmsnorm_bwd(torch.from_numpy(dy64), xs, w, eps, want_dw=False)
        _, rr = oracle.rmsnorm_fwd(xs, None, eps)
        gg = np.abs(dy64 * to64(w)[None, :])
        xh = np.abs(to64(xs) * rr[:, None])
        extra = (2 ** -8) * 1.01 * rr[:, None] * (gg + xh * np.mean(gg * xh, axis=1, keepdims=True))
        check(f"chain bwd dx rows {b0}..", dx[b0:b1], rdx, "bf16", extra=extra, s=grad_scale(rr, dy64, w))


# ---------------------------------------------------------------- edge cases

NORM_EDGES = [
    # (rows, n, dtype)
    (1, 1, torch.float32), (3, 7, torch.bfloat16), (257, 64, torch.float32),
    (5, 255, torch.bfloat16), (64, 256, torch.bfloat16), (33, 1000, torch.float32),
    (17, 5128, torch.bfloat16), (9, 8191, torch.bfloat16), (4, 12288, torch.float32),
    (3, 32768, torch.float32), (3, 65536, torch.bfloat16), (1000, 40, torch.bfloat16),
    # IEEE fp16 storage
    (7, 40, torch.float16), (33, 1000, torch.float16), (65, 5120, torch.float16),
    (5, 4097, torch.float16), (2, 65536, torch.float16),
    # rows past 16384 elements: RMSNorm's one-pass backward with its dW
    # accumulators in LDS (aligned 16-bit rows up to 32768: 20480, 16392 and
    # 32768, the last two with many rows per workgroup), and the two-pass
    # backward (element-wise 17001, fp32 24576, LayerNorm throughout)
    (37, 20480, torch.bfloat16), (5, 17001, torch.float16), (9, 24576, torch.float32),
    (300, 16392, torch.float16), (600, 32768, torch.bfloat16),
    # batches of 3584..4096 rows, where the RMSNorm forward packs eight row
    # groups (16 rows) into a workgroup; a partial last workgroup included
    (4095, 4104, torch.bfloat16), (3584, 2560, torch.float32), (3601, 5000, torch.float16),
    # narrow rows on many rows: two to four backward workgroups per CU
    (15000, 1280, torch.bfloat16), (9001, 2560, torch.float16), (8200, 2048, torch.bfloat16),
    # per-head-sized rows on many rows: two rows a wave forward, up to eight
    # backward workgroups per CU
    (40003, 128, torch.bfloat16), (20000, 256, torch.float32), (17000, 256, torch.float16),
]


@pytest.mark.parametrize("rows,n,dtype", NORM_EDGES)
@pytest.mark.parametrize("gemma", [False, True])
def test_rms_edges(rows, n, dtype, gemma):
    seed = 2000 + rows * 7 + n
    x = workloads.normal((rows, n), seed, dtype)
    w = workloads.normal((n,), seed + 1, dtype, std=0.1, mean=0.0 if gemma else 1.0)
    dy = workloads.normal((rows, n), seed + 2, dtype)
    check_rms_full(f"rms edge {rows}x{n}", x, w, dy, 1e-6, gemma)


@pytest.mark.parametrize("rows,n,dtype", NORM_EDGES)
def test_ln_edges(rows, n, dtype):
    seed = 3000 + rows * 7 + n
    x = workloads.normal((rows, n), seed, dtype, mean=0.5, std=2.0)
    gm = workloads.normal((n,), seed + 1, dtype, mean=1.0, std=0.1)
    bt = workloads.normal((n,), seed + 2, dtype, std=0.1)
    dy = workloads.normal((rows, n), seed + 3, dtype)
    check_ln_full(f"ln edge {rows}x{n}", x, gm, bt, dy, 1e-5)


# Forwards of aligned rows of at most 32 16-byte chunks put 64 / S rows side
# by side in a wave, S lanes each.  Each lane width, forced, on ragged batches
# (a partial last wave and workgroup), rows that leave lanes of their S idle,
# and every operator and epilogue of the forward, against the oracle.
PACKED = [
    # (S, rows, n, dtype)
    (4, 1037, 24, torch.bfloat16), (4, 3, 16, torch.float32), (8, 1001, 64, torch.bfloat16),
    (8, 517, 28, torch.float32), (16, 1039, 120, torch.float16), (16, 2050, 128, torch.bfloat16),
    (32, 1, 256, torch.bfloat16), (32, 777, 200, torch.bfloat16), (32, 1030, 128, torch.float32),
    (32, 300, 64, torch.bfloat16),  # 8 chunks on 32 lanes
]


class forced_pack:
    def __init__(self, s):
        self.s = s

    def __enter__(self):
        nr.nr_tune("fwd_pack", self.s)

    def __exit__(self, *a):
        nr.nr_tune("fwd_pack", 0)


@pytest.mark.parametrize("S,rows,n,dtype", PACKED)
@pytest.mark.parametrize("op", ["rms", "rms_gemma", "ln", "ln_gelu", "rms_rope"])
def test_packed_rows_forward(S, rows, n, dtype, op):
    seed = 9100 + S * 13 + rows + n
    say(f"packed forward S={S} {rows}x{n} {dtype} {op}")
    x = workloads.normal((rows, n), seed, dtype, mean=0.5 if op.startswith("ln") else 0.0, std=2.0)
    gemma = op == "rms_gemma"
    w = workloads.normal((n,), seed + 1, dtype, mean=0.0 if gemma else 1.0, std=0.1)
    k = out_kind(dtype)
    with forced_pack(S):
        if op in ("rms", "rms_gemma"):
            y, r = nr.rmsnorm_fwd(g(x), g(w), eps=1e-6, gemma_offset=gemma)
            torch.cuda.synchronize()
            ry, rr = oracle.rmsnorm_fwd(x, w, 1e-6, gemma)
            check(f"S={S} y", y.reshape(-1, n), ry, k)
            check(f"S={S} inv_rms", r.reshape(-1), rr, "stat", s=0.0)
        elif op == "rms_rope":
            hd = n if n % 16 else n // 2  # per-head rows, or two heads a row
            rpt = 2 if hd == n else 1
            ang = oracle.rope_angles_1d(-(-rows // rpt), hd, 5, 10000.0)
            ct = torch.from_numpy(np.cos(ang)).float().to("cuda")
            st = torch.from_numpy(np.sin(ang)).float().to("cuda")
            y, r = nr.rmsnorm_rope_fwd(g(x), g(w), ct, st, hd, rpt, 1e-6, False)
            torch.cuda.synchronize()
            ry, rr = oracle.rmsnorm_rope_fwd(x, w, ang, hd, rpt, 1e-6, False)
            check(f"S={S} y", y, ry, k)
            check(f"S={S} inv_rms", r, rr, "stat", s=0.0)
        else:
            bt = workloads.normal((n,), seed + 2, dtype, std=0.5)
            x64 = to64(x).reshape(-1, n)
            if op == "ln":
                y, mu, rs = nr.layernorm_fwd(g(x), g(w), g(bt), eps=1e-5)
                ry, rmu, rrs = oracle.layernorm_fwd(x, w, bt, 1e-5)
            else:
                y, mu, rs = nr.layernorm_gelu_fwd(g(x), g(w), g(bt), 1e-5)
                ry, rmu, rrs = oracle.layernorm_gelu_fwd(x, w, bt, 1e-5)
            torch.cuda.synchronize()
            check(f"S={S} y", y.reshape(-1, n), ry, k)
            check(f"S={S} mean", mu.reshape(-1), rmu, "stat", s=np.sqrt(np.mean(x64 * x64, axis=1)))
            check(f"S={S} rstd", rs.reshape(-1), rrs, "stat", s=0.0)


class forced_bwd_pack(forced_pack):
    def __enter__(self):
        nr.nr_tune("bwd_pack", self.s)

    def __exit__(self, *a):
        nr.nr_tune("bwd_pack", 0)


@pytest.mark.parametrize("S,rows,n,dtype", PACKED)
@pytest.mark.parametrize("op", ["rms", "rms_gemma", "rms_no_weight", "ln", "rms_rope", "ln_gelu"])
def test_packed_rows_backward(S, rows, n, dtype, op):
    """The backward's packed form (S lanes a row, column sums through LDS and
    the column reduction), each lane width forced, against the oracle."""
    seed = 9500 + S * 13 + rows + n
    say(f"packed backward S={S} {rows}x{n} {dtype} {op}")
    x = workloads.normal((rows, n), seed, dtype, mean=0.5 if op.startswith("ln") else 0.0, std=2.0)
    gemma = op == "rms_gemma"
    w = workloads.normal((n,), seed + 1, dtype, mean=0.0 if gemma else 1.0, std=0.1)
    dy = workloads.normal((rows, n), seed + 2, dtype)
    with forced_bwd_pack(S):
        if op == "ln":
            bt = workloads.normal((n,), seed + 3, dtype, std=0.5)
            check_ln_full(f"S={S}", x, w, bt, dy, 1e-5)
        elif op == "ln_gelu":
            bt = workloads.normal((n,), seed + 3, dtype, std=0.5)
            _, mu, rs = nr.layernorm_gelu_fwd(g(x), g(w), g(bt), 1e-5)
            dx, dg, db = nr.layernorm_gelu_bwd(g(dy), g(x), g(w), g(bt), mu, rs)
            torch.cuda.synchronize()
            rdx, rdg, rdb = oracle.layernorm_gelu_bwd(dy, x, w, bt, 1e-5)
            _, _, rrs = oracle.layernorm_gelu_fwd(x, w, bt, 1e-5)
            # |gelu'| stays below 1.13
            check(f"S={S} dx", dx, rdx, out_kind(dtype), s=1.13 * grad_scale(rrs, dy, w))
            check(f"S={S} dgamma", dg, rdg, "col")
            check(f"S={S} dbeta", db, rdb, "col")
        elif op == "rms_rope":
            hd = n if n % 16 else n // 2
            rpt = 2 if hd == n else 1
            ang = oracle.rope_angles_1d(-(-rows // rpt), hd, 5, 10000.0)
            ct = torch.from_numpy(np.cos(ang)).float().to("cuda")
            st = torch.from_numpy(np.sin(ang)).float().to("cuda")
            y, r = nr.rmsnorm_rope_fwd(g(x), g(w), ct, st, hd, rpt, 1e-6, False)
            dx, dw = nr.rmsnorm_rope_bwd(g(dy), g(x), g(w), r, ct, st, hd, rpt, False)
            torch.cuda.synchronize()
            rdx, rdw = oracle.rmsnorm_rope_bwd(dy, x, w, ang, hd, rpt, 1e-6, False)
            _, rr = oracle.rmsnorm_rope_fwd(x, w, ang, hd, rpt, 1e-6, False)
            dy64 = oracle.rope_apply(dy.reshape(1, rows, n // hd, hd),
                                     ang[np.arange(rows) // rpt], inverse=True).reshape(rows, n)
            check(f"S={S} dx", dx, rdx, out_kind(dtype), s=grad_scale(rr, dy64, w, False))
            check(f"S={S} dw", dw, rdw, "col")
        else:
            check_rms_full(f"S={S}", x, None if op == "rms_no_weight" else w, dy, 1e-6, gemma)


def test_non_affine_and_constant_rows():
    x = workloads.normal((40, 96), 4001, torch.bfloat16)
    dy = workloads.normal((40, 96), 4002, torch.bfloat16)
    check_rms_full("rms no weight", x, None, dy, 1e-6, False)
    x[3] = 1.5  # constant row: LayerNorm gives beta (zero deviation)
    check_ln_full("ln no gamma/beta", x, None, None, dy, 1e-5)
    bt = workloads.normal((96,), 4003, torch.bfloat16)
    say("ln constant row")
    y, _, _ = nr.layernorm_fwd(g(x), None, g(bt), eps=1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y[3].cpu(), bt)


def test_in_place_and_unaligned():
    rows, n = 70, 520
    x = workloads.normal((rows, n), 4100, torch.bfloat16)
    w = workloads.normal((n,), 4101, torch.bfloat16, mean=1.0, std=0.1)
    dy = workloads.normal((rows, n), 4102, torch.bfloat16)
    ry, _ = oracle.rmsnorm_fwd(x, w, 1e-6)
    rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
    say("rms in place y == x, dx == dy")
    xg = g(x)
    _, r = nr.rmsnorm_fwd(g(x), g(w), eps=1e-6)
    dyg = g(dy)
    nr.rmsnorm_bwd(dyg, xg, g(w), r, dx=dyg)
    nr.rmsnorm_fwd(xg, g(w), eps=1e-6, y=xg)
    torch.cuda.synchronize()
    check("in-place y", xg, ry, "bf16")
    check("in-place dx", dyg, rdx, "bf16")
    say("rms unaligned rows (element-wise path)")
    buf = torch.empty(rows * n + 1, dtype=torch.bfloat16, device=DEV)
    xu = buf[1:].view(rows, n)
    xu.copy_(g(x))
    buf2 = torch.empty(rows * n + 3, dtype=torch.bfloat16, device=DEV)
    yu = buf2[3:].view(rows, n)
    _, ru = nr.rmsnorm_fwd(xu, g(w), eps=1e-6, y=yu)
    dbuf = torch.empty(rows * n + 1, dtype=torch.bfloat16, device=DEV)
    dyu = dbuf[1:].view(rows, n)
    dyu.copy_(g(dy))
    dxu, dwu = nr.rmsnorm_bwd(dyu, xu, g(w), ru)
    torch.cuda.synchronize()
    check("unaligned y", yu, ry, "bf16")
    check("unaligned dx", dxu, rdx, "bf16")
    check("unaligned dw", dwu, rdw, "col")


def test_empty_batch():
    say("rows == 0")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y, r = nr.rmsnorm_fwd(x, w)
    dw = torch.full((64,), 7.0, device=DEV)
    nr.rmsnorm_bwd(x, x, w, r, dw=dw)
    dg = torch.full((64,), 7.0, device=DEV)
    db = torch.full((64,), 7.0, device=DEV)
    _, mu, rs = nr.layernorm_fwd(x, w, w)
    nr.layernorm_bwd(x, x, w, mu, rs, dgamma=dg, dbeta=db)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)
    assert torch.all(dw == 0) and torch.all(dg == 0) and torch.all(db == 0)


@pytest.mark.parametrize("kind", ["rms", "ln", "ln_gelu", "rms_rope"])
def test_backward_bitwise_deterministic(kind):
    # every backward, the fused ones included (the GeLU one adds its wave
    # sums in a DPP tree, the LayerNorm, GeLU and RoPE ones read their row
    # statistics through scalar loads): bit-identical results on repeat
    inp = workloads.norm_inputs("rms_gemma_3840x5120")
    x, w, dy = g(inp["x"]), g(inp["w"]), g(inp["dy"])
    say(f"{kind} bwd determinism 3840x5120")
    ct, st = nr.rope_table_1d(x.shape[0], 128, 0, 10000.0, device=DEV)
    outs = []
    for _ in range(2):
        if kind == "rms":
            _, r = nr.rmsnorm_fwd(x, w, gemma_offset=True)
            outs.append(nr.rmsnorm_bwd(dy, x, w, r, gemma_offset=True))
        elif kind == "ln":
            _, mu, rs = nr.layernorm_fwd(x, w, w)
            outs.append(nr.layernorm_bwd(dy, x, w, mu, rs))
        elif kind == "ln_gelu":
            _, mu, rs = nr.layernorm_gelu_fwd(x, w, w)
            outs.append(nr.layernorm_gelu_bwd(dy, x, w, w, mu, rs))
        else:
            _, r = nr.rmsnorm_rope_fwd(x, w, ct, st, 128)
            outs.append(nr.rmsnorm_rope_bwd(dy, x, w, r, ct, st, 128))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kind,n", [("rms", 20480), ("rms", 40960), ("ln", 20480)])
def test_long_row_backward_deterministic_and_without_column_gradients(kind, n):
    # RMSNorm 20480: one pass, dW in LDS (38 workgroups of 8 rows); RMSNorm
    # 40960 and LayerNorm: two passes (19 row groups)
    rows = 300
    x = workloads.normal((rows, n), 6100, torch.bfloat16)
    w = workloads.normal((n,), 6101, torch.bfloat16, mean=1.0, std=0.1)
    dy = workloads.normal((rows, n), 6102, torch.bfloat16)
    say(f"{kind} long-row bwd determinism {rows}x{n}")
    xg, wg, dyg = g(x), g(w), g(dy)
    outs = []
    for _ in range(2):
        if kind == "rms":
            _, r = nr.rmsnorm_fwd(xg, wg)
            outs.append(nr.rmsnorm_bwd(dyg, xg, wg, r))
        else:
            _, mu, rs = nr.layernorm_fwd(xg, wg, wg)
            outs.append(nr.layernorm_bwd(dyg, xg, wg, mu, rs))
    # dx alone (the workspace still carries the row terms)
    if kind == "rms":
        dx_only, none = nr.rmsnorm_bwd(dyg, xg, wg, r, want_dw=False)
        assert none is None
    else:
        dx_only, n1, n2 = nr.layernorm_bwd(dyg, xg, wg, mu, rs, want_dgamma=False, want_dbeta=False)
        assert n1 is None and n2 is None
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    assert torch.equal(dx_only, outs[0][0])
    if kind == "rms":
        rdx, rdw = oracle.rmsnorm_bwd(dy, x, w, 1e-6)
        _, rr = oracle.rmsnorm_fwd(x, w, 1e-6)
        check("long rms dx", outs[0][0], rdx, "bf16", s=grad_scale(rr, dy, w))
        check("long rms dw", outs[0][1], rdw, "col")
    else:
        rdx, rdg, rdb = oracle.layernorm_bwd(dy, x, w, 1e-5)
        _, _, rrs = oracle.layernorm_fwd(x, w, w, 1e-5)
        check("long ln dx", outs[0][0], rdx, "bf16", s=grad_scale(rrs, dy, w))
        check("long ln dgamma", outs[0][1], rdg, "col")
        check("long ln dbeta", outs[0][2], rdb, "col")


ROPE_EDGES = [
    # (batch, tokens, heads, head_dim, dtype, layout)
    (1, 5, 1, 2, torch.float32, "packed"),
    (2, 9, 3, 6, torch.bfloat16, "packed"),
    (1, 33, 40, 128, torch.bfloat16, "packed"),
    (2, 17, 8, 64, torch.float32, "packed"),
    (1, 12, 5, 256, torch.bfloat16, "packed"),
    (1, 7, 96, 128, torch.bfloat16, "packed"),       # several passes over the heads
    (2, 10, 4, 64, torch.bfloat16, "bhtd"),          # heads-major storage, strided view
    (1, 11, 3, 32, torch.float32, "unaligned"),      # element-wise path
    (1, 13, 2, 10, torch.bfloat16, "padded"),        # head stride > head_dim
    (1, 33, 40, 128, torch.float16, "packed"),
    (2, 9, 3, 34, torch.float16, "unaligned"),
]


@pytest.mark.parametrize("b,t,h,d,dtype,layout", ROPE_EDGES)
def test_rope_edges(b, t, h, d, dtype, layout):
    x = workloads.normal((b, t, h, d), 5000 + t * h + d, dtype)
    pos0 = 1000 if layout == "padded" else 0
    ang = oracle.rope_angles_1d(t, d, pos0, 10000.0)
    say(f"rope edge {b}x{t}x{h}x{d} {dtype} {layout}")
    ct, st = nr.rope_table_1d(t, d, pos0, 10000.0)
    for inv in (False, True):
        if layout == "packed":
            xg = g(x).clone()
        elif layout == "bhtd":
            xg = g(x).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        elif layout == "unaligned":
            buf = torch.empty(x.numel() + 1, dtype=dtype, device=DEV)
            xg = buf[1:].view(x.shape)
            xg.copy_(g(x))
        else:
            buf = torch.zeros((b, t, h, d + 6), dtype=dtype, device=DEV)
            xg = buf[..., :d]
            xg.copy_(g(x))
        nr.rope_interleaved_apply(xg, ct, st, inverse=inv)
        torch.cuda.synchronize()
        if layout == "padded":
            assert torch.all(buf[..., d:] == 0), "rope wrote outside the head vectors"
        ref = oracle.rope_apply(x, ang, inv)
        check(f"rope edge {layout} inv={inv}", xg.reshape(-1, d), ref.reshape(-1, d), out_kind(dtype))


def test_rope_table_3d_small():
    spec = dict(kind="3d", grid=(3, 4, 5), pairs=(5, 4, 3), theta=10000.0)
    say("rope 3-D table 3x4x5 pairs 5/4/3")
    ct, st = gpu_table(spec, 60, 24)
    torch.cuda.synchronize()
    check_table("3d small", ct, st, oracle.rope_angles(spec, 60, 24))


def test_errors_raise():
    x = torch.zeros((2, 3, 4, 7), dtype=torch.bfloat16, device=DEV)
    c = torch.zeros((3, 3), device=DEV)
    with pytest.raises((nr.NormRopeError, ValueError)):
        nr.rope_interleaved_apply(x, c, c)
    with pytest.raises(nr.NormRopeError):
        nr.rmsnorm_fwd(torch.zeros((2, 70000), dtype=torch.bfloat16, device=DEV))
