"""Benchmark: achieved HBM bandwidth of the fused norm fwd+bwd and RoPE path.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step runs every operation of the path once over one batch that is
already resident in HBM, by default on the long-sequence workload
(x [65536, 5120] bf16, viewed as 65536 tokens x 40 heads x 128 for RoPE):

  rmsnorm_fwd(x) -> y, inv_rms        rope forward on y (in place)
  rope inverse on dout (in place)     rmsnorm_bwd(dout, x) -> dx, dw
  layernorm_fwd(x) -> y2, mean, rstd  layernorm_bwd(dout, x) -> dx2, dgamma, dbeta

The cos/sin table is built once per shape, outside the steps.  `value` is
the algorithmic bytes of one step (each tensor read or written once; weights
once per call; statistics and column gradients in fp32; no workspace) divided
by the measured time per step.  The other workloads (--workload) time their
own operations the same way.  One JSON line goes to stdout.

After the timed steps, outside them: the library's streaming copy over one
65536 x 5120 bf16 activation gives the practical HBM ceiling ("ceiling";
the roofline also reports its fraction of it), and each operation is timed
alone --cold-rounds times with the caches flushed before every call
("ops_cold": mean, std, min).

--copy-probe runs only a plain device copy of known size: the reference the
HBM byte counters are scaled by.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (and % of peak) for fused norm fwd+bwd and RoPE"
PEAK_GBS = 8000.0  # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "rmsnorm_layernorm_fwd_amd", "csrc")


# ---------------------------------------------------------------- bytes

def rms_fwd_bytes(m, n, e=2):
    return 2 * e * m * n + e * n + 4 * m


def rms_bwd_bytes(m, n, e=2):
    return 3 * e * m * n + e * n + 4 * m + 4 * n


def ln_fwd_bytes(m, n, e=2):
    return 2 * e * m * n + 2 * e * n + 8 * m


def ln_bwd_bytes(m, n, e=2):
    return 3 * e * m * n + e * n + 8 * m + 8 * n


def rope_bytes(t, h, d, e=2):
    return 2 * e * t * h * d + 2 * 4 * t * (d // 2)


def source_hash(workload=None):
    """Hash of the library sources the workload's kernels are compiled from:
    counter summaries taken on other sources are not reused.  The folded
    RMSNorm->linear kernel has a source file of its own (plus the two shared
    headers); the row and RoPE kernels are built from everything else."""
    gemm = workload is not None and workload.startswith(("rms_linear", "ln_linear"))
    hsh = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if not f.endswith((".hip", ".hpp")):
            continue
        if gemm and f not in ("gemm_rmsnorm.hip", "nr_device.hpp", "nr_internal.hpp"):
            continue
        if workload is not None and not gemm and f == "gemm_rmsnorm.hip":
            continue
        with open(os.path.join(CSRC, f), "rb") as fh:
            hsh.update(f.encode() + fh.read())
    return hsh.hexdigest()[:16]


# ---------------------------------------------------------------- workloads

def build_ops(name, dev):
    """Returns (ops, description): ops = [(label, kernel_name, fn, bytes)]."""
    import torch

    import rmsnorm_layernorm_fwd_amd as nr
    import workloads

    g = lambda t: None if t is None else t.to(dev)
    ops = []
    if name == "longseq_65536x5120":
        inp = workloads.norm_inputs(name)
        ln_params = workloads.norm_inputs("ln_affine_15360x5120")
        m, n = inp["x"].shape
        h, d = 40, 128
        x, w, dout = g(inp["x"]), g(inp["w"]), g(inp["dy"])
        gm, bt = g(ln_params["w"]), g(ln_params["b"])
        y, dx, y2, dx2 = (torch.empty_like(x) for _ in range(4))
        r = torch.empty(m, dtype=torch.float32, device=dev)
        mu, rs = torch.empty_like(r), torch.empty_like(r)
        dw, dg, db = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3))
        ws = torch.empty(max(nr.nr_bwd_workspace_bytes(m, n, 1), 16), dtype=torch.uint8, device=dev)
        ct, st = nr.rope_table_1d(m, d, 0, 10000.0, device=dev)
        yv, gv = y.view(1, m, h, d), dout.view(1, m, h, d)
        ops = [
            ("rmsnorm_fwd", "norm_fwd[rms]", lambda: nr.rmsnorm_fwd(x, w, 1e-6, y=y, inv_rms=r),
             rms_fwd_bytes(m, n)),
            ("rope_fwd", "rope_apply_kernel", lambda: nr.rope_interleaved_apply(yv, ct, st),
             rope_bytes(m, h, d)),
            ("rope_inverse", "rope_apply_kernel",
             lambda: nr.rope_interleaved_apply(gv, ct, st, inverse=True), rope_bytes(m, h, d)),
            ("rmsnorm_bwd", "norm_bwd_rows[rms]+colreduce",
             lambda: nr.rmsnorm_bwd(dout, x, w, r, dx=dx, dw=dw, workspace=ws), rms_bwd_bytes(m, n)),
            ("layernorm_fwd", "norm_fwd[ln]",
             lambda: nr.layernorm_fwd(x, gm, bt, 1e-5, y=y2, mean=mu, rstd=rs), ln_fwd_bytes(m, n)),
            ("layernorm_bwd", "norm_bwd_rows[ln]+colreduce",
             lambda: nr.layernorm_bwd(dout, x, gm, mu, rs, dx=dx2, dgamma=dg, dbeta=db, workspace=ws),
             ln_bwd_bytes(m, n)),
        ]
        desc = dict(workload=name, rows=m, hidden=n, heads=h, head_dim=d, io_dtype="bf16",
                    positions="1-D 0..65535, theta 1e4", rms_eps=1e-6, ln_eps=1e-5,
                    outlier_rows=int(len(inp["outlier_rows"])))
    elif name == "longseq_fused_65536x5120":
        # the long-sequence norm -> RoPE chain with the fused kernels: one
        # read and one write of the row per direction
        inp = workloads.norm_inputs("longseq_65536x5120")
        m, n = inp["x"].shape
        h, d = 40, 128
        x, w, dout = g(inp["x"]), g(inp["w"]), g(inp["dy"])
        y, dx = torch.empty_like(x), torch.empty_like(x)
        r = torch.empty(m, dtype=torch.float32, device=dev)
        dw = torch.empty(n, dtype=torch.float32, device=dev)
        ws = torch.empty(max(nr.nr_bwd_workspace_bytes(m, n, 2), 16), dtype=torch.uint8, device=dev)
        ct, st = nr.rope_table_1d(m, d, 0, 10000.0, device=dev)
        tab = 2 * 4 * m * (d // 2)
        ops = [
            ("rmsnorm_rope_fwd", "norm_fwd[rms+rope]",
             lambda: nr.rmsnorm_rope_fwd(x, w, ct, st, d, 1, 1e-6, y=y, inv_rms=r), rms_fwd_bytes(m, n) + tab),
            ("rmsnorm_rope_bwd", "norm_bwd_rows[rms+rope]+colreduce",
             lambda: nr.rmsnorm_rope_bwd(dout, x, w, r, ct, st, d, 1, dx=dx, dw=dw, workspace=ws),
             rms_bwd_bytes(m, n) + tab),
        ]
        desc = dict(workload=name, rows=m, hidden=n, heads=h, head_dim=d, io_dtype="bf16",
                    positions="1-D 0..65535, theta 1e4", rms_eps=1e-6)
    elif name == "rms_gemma_3840x5120":
        inp = workloads.norm_inputs(name)
        m, n = inp["x"].shape
        x, w, dy = g(inp["x"]), g(inp["w"]), g(inp["dy"])
        y, dx = torch.empty_like(x), torch.empty_like(x)
        r = torch.empty(m, dtype=torch.float32, device=dev)
        dw = torch.empty(n, dtype=torch.float32, device=dev)
        ws = torch.empty(max(nr.nr_bwd_workspace_bytes(m, n, 0), 16), dtype=torch.uint8, device=dev)
        ops = [
            ("rmsnorm_fwd", "norm_fwd[rms]",
             lambda: nr.rmsnorm_fwd(x, w, 1e-6, True, y=y, inv_rms=r), rms_fwd_bytes(m, n)),
            ("rmsnorm_bwd", "norm_bwd_rows[rms]+colreduce",
             lambda: nr.rmsnorm_bwd(dy, x, w, r, True, dx=dx, dw=dw, workspace=ws), rms_bwd_bytes(m, n)),
        ]
        desc = dict(workload=name, rows=m, hidden=n, io_dtype="bf16", gemma_offset=True)
    elif name == "ln_affine_15360x5120":
        inp = workloads.norm_inputs(name)
        m, n = inp["x"].shape
        x, gm, bt, dy = g(inp["x"]), g(inp["w"]), g(inp["b"]), g(inp["dy"])
        y, dx = torch.empty_like(x), torch.empty_like(x)
        mu = torch.empty(m, dtype=torch.float32, device=dev)
        rs = torch.empty_like(mu)
        dg, db = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2))
        ws = torch.empty(max(nr.nr_bwd_workspace_bytes(m, n, 1), 16), dtype=torch.uint8, device=dev)
        ops = [
            ("layernorm_fwd", "norm_fwd[ln]",
             lambda: nr.layernorm_fwd(x, gm, bt, 1e-5, y=y, mean=mu, rstd=rs), ln_fwd_bytes(m, n)),
            ("layernorm_bwd", "norm_bwd_rows[ln]+colreduce",
             lambda: nr.layernorm_bwd(dy, x, gm, mu, rs, dx=dx, dgamma=dg, dbeta=db, workspace=ws),
             ln_bwd_bytes(m, n)),
        ]
        desc = dict(workload=name, rows=m, hidden=n, io_dtype="bf16")
    elif name == "ln_gelu_15360x5120":
        inp = workloads.norm_inputs("ln_affine_15360x5120")
        m, n = inp["x"].shape
        x, gm, bt, dy = g(inp["x"]), g(inp["w"]), g(inp["b"]), g(inp["dy"])
        y, dx = torch.empty_like(x), torch.empty_like(x)
        mu = torch.empty(m, dtype=torch.float32, device=dev)
        rs = torch.empty_like(mu)
        dg, db = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(2))
        ws = torch.empty(max(nr.nr_bwd_workspace_bytes(m, n, 1), 16), dtype=torch.uint8, device=dev)
        ops = [
            ("layernorm_gelu_fwd", "norm_fwd[ln+gelu]",
             lambda: nr.layernorm_gelu_fwd(x, gm, bt, 1e-5, y=y, mean=mu, rstd=rs), ln_fwd_bytes(m, n)),
            ("layernorm_gelu_bwd", "ln_gelu_bwd_pair+colreduce",
             lambda: nr.layernorm_gelu_bwd(dy, x, gm, bt, mu, rs, dx=dx, dgamma=dg, dbeta=db, workspace=ws),
             ln_bwd_bytes(m, n) + 2 * n),
        ]
        desc = dict(workload=name, rows=m, hidden=n, io_dtype="bf16", activation="tanh-GeLU")
    elif name == "rope3d_15360x40x128":
        inp = workloads.rope_inputs(name)
        b, t, h, d = inp["shape"]
        q, k = g(inp["q"]), g(inp["k"])
        ct, st = nr.rope_table_3d(inp["table"]["grid"], inp["table"]["pairs"], 10000.0, device=dev)
        ops = [
            ("rope_fwd_q", "rope_apply_kernel", lambda: nr.rope_interleaved_apply(q, ct, st), rope_bytes(t, h, d)),
            ("rope_fwd_k", "rope_apply_kernel", lambda: nr.rope_interleaved_apply(k, ct, st), rope_bytes(t, h, d)),
            ("rope_inverse_q", "rope_apply_kernel",
             lambda: nr.rope_interleaved_apply(q, ct, st, inverse=True), rope_bytes(t, h, d)),
            ("rope_inverse_k", "rope_apply_kernel",
             lambda: nr.rope_interleaved_apply(k, ct, st, inverse=True), rope_bytes(t, h, d)),
        ]
        desc = dict(workload=name, tokens=t, heads=h, head_dim=d, io_dtype="bf16",
                    positions="3-D 16x24x40, pairs 22/21/21, theta 1e4")
    elif name == "rms_linear_65536x5120x5120":
        # RMSNorm folded into the following linear layer (a 5120 -> 5120
        # projection of the long-sequence activation): matrix-core bound
        inp = workloads.norm_inputs("longseq_65536x5120")
        m, k = inp["x"].shape
        n = 5120
        x, w = g(inp["x"]), g(inp["w"])
        W = workloads.normal((n, k), 4242, torch.bfloat16, std=k ** -0.5).to(dev)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        r = torch.empty(m, dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, nr.nr_rmsnorm_linear_workspace_bytes(m, n, k, True)),
                         dtype=torch.uint8, device=dev)
        # one call: the norm weight folded into W (a 52 MB pass), then the
        # GEMM kernel; the call's time, fold included, is charged to the GEMM
        ops = [
            ("rmsnorm_linear_fwd", "norm_linear_tile256_kernel[rms]",
             lambda: nr.rmsnorm_linear_fwd(x, w, W, 1e-6, out=out, inv_rms=r, workspace=ws),
             2 * m * k + 2 * n * k + 2 * k + 2 * m * n + 4 * m),
        ]
        y = torch.empty_like(x)
        desc = dict(workload=name, rows=m, hidden=k, out_features=n, io_dtype="bf16",
                    flops_per_step=2 * m * n * k, weight="W ~ N(0, 1/K), seed 4242",
                    unfused=dict(fns=[lambda: nr.rmsnorm_fwd(x, w, 1e-6, y=y, inv_rms=r),
                                      lambda: torch.matmul(y, W.t(), out=out)],
                                 what="rmsnorm_fwd, then torch.matmul (the vendor GEMM) on y"))
    elif name == "ln_linear_65536x5120x5120":
        # LayerNorm folded into the following linear layer (a 5120 -> 5120
        # projection of the long-sequence activation, with the affine
        # LayerNorm parameters): matrix-core bound
        inp = workloads.norm_inputs("longseq_65536x5120")
        lnp = workloads.norm_inputs("ln_affine_15360x5120")
        m, k = inp["x"].shape
        n = 5120
        x, gm, bt = g(inp["x"]), g(lnp["w"]), g(lnp["b"])
        W = workloads.normal((n, k), 4243, torch.bfloat16, std=k ** -0.5).to(dev)
        out = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
        mu, rs = (torch.empty(m, dtype=torch.float32, device=dev) for _ in range(2))
        ws = torch.empty(max(1, nr.nr_layernorm_linear_workspace_bytes(m, n, k, True)),
                         dtype=torch.uint8, device=dev)
        # one call: row statistics, the fold (a 52 MB pass) and the GEMM; the
        # call's whole time is charged to the GEMM
        ops = [
            ("layernorm_linear_fwd", "norm_linear_tile256_kernel[ln]",
             lambda: nr.layernorm_linear_fwd(x, gm, bt, W, 1e-5, out=out, mean=mu, rstd=rs,
                                             workspace=ws),
             2 * m * k + 2 * n * k + 4 * k + 2 * m * n + 8 * m),
        ]
        y = torch.empty_like(x)
        desc = dict(workload=name, rows=m, hidden=k, out_features=n, io_dtype="bf16",
                    flops_per_step=2 * m * n * k, weight="W ~ N(0, 1/K), seed 4243",
                    unfused=dict(fns=[lambda: nr.layernorm_fwd(x, gm, bt, 1e-5, y=y, mean=mu, rstd=rs),
                                      lambda: torch.matmul(y, W.t(), out=out)],
                                 what="layernorm_fwd, then torch.matmul (the vendor GEMM) on y"))
    else:
        raise SystemExit(f"unknown workload {name}")
    return ops, desc


def time_fns(fns, reps=10):
    """Mean milliseconds of one pass over fns (events on the launch stream)."""
    import torch

    for _ in range(3):
        for f in fns:
            f()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        for f in fns:
            f()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


# ---------------------------------------------------------------- traffic

def read_traffic(kernel_label, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    missing or taken on different kernel sources."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_hash") != source_hash(workload):
        return None
    # a label "a[..]+b" names kernels launched together (the backward's rows
    # and its column reduction): their bytes add; "+" inside [] is a name
    parts, depth, cur = [], 0, ""
    for ch in kernel_label:
        depth += (ch == "[") - (ch == "]")
        if ch == "+" and depth == 0:
            parts.append(cur)
            cur = ""
        else:
            cur += ch
    parts.append(cur)
    vals = [kv.get(f"bytes_per_launch.{p}") for p in parts]
    return float(sum(float(v) for v in vals)) if all(vals) else None


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(seconds):
    """The fp64 oracle, as it stands, on the host cores: the same step on the
    first rows of the long-sequence workload, repeated for about `seconds`."""
    import torch

    import oracle
    import workloads

    rows = 1024
    inp = workloads.norm_inputs("longseq_65536x5120")
    lnp = workloads.norm_inputs("ln_affine_15360x5120")
    x, w, dy = inp["x"][:rows].clone(), inp["w"], inp["dy"][:rows].clone()
    gm, bt = lnp["w"], lnp["b"]
    n, h, d = x.shape[1], 40, 128
    ang = oracle.rope_angles_1d(rows, d, 0, 10000.0)
    per_pass = (rms_fwd_bytes(rows, n) + 2 * rope_bytes(rows, h, d) + rms_bwd_bytes(rows, n)
                + ln_fwd_bytes(rows, n) + ln_bwd_bytes(rows, n))
    oracle.lib()
    passes, t0 = 0, time.perf_counter()
    while True:
        y, _ = oracle.rmsnorm_fwd(x, w, 1e-6)
        oracle.rope_apply(torch.from_numpy(y).view(1, rows, h, d), ang)
        oracle.rope_apply(dy.view(1, rows, h, d), ang, inverse=True)
        oracle.rmsnorm_bwd(dy, x, w, 1e-6)
        oracle.layernorm_fwd(x, gm, bt, 1e-5)
        oracle.layernorm_bwd(dy, x, gm, 1e-5)
        passes += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    cores = oracle.max_threads()
    return dict(value=round(per_pass * passes / el / 1e9, 4), unit="GB/s", cores=cores,
                host_cpus=os.cpu_count(), omp_max_threads=cores, kind="oracle",
                sample=(f"the long-sequence step (rmsnorm fwd, rope fwd, rope inverse, rmsnorm bwd, "
                        f"layernorm fwd, layernorm bwd) on rows 0..{rows - 1} of 65536, {passes} passes "
                        f"in {el:.1f} s, fp64, OpenMP over rows; bytes counted as for the GPU"))


# ---------------------------------------------------------------- main

def stream_ceiling(dev, reps=10):
    """The practical HBM ceiling: the library's streaming copy (the row
    kernels' access pattern, no arithmetic) over one activation of the
    long-sequence size, 65536 x 5120 bf16."""
    import torch

    import rmsnorm_layernorm_fwd_amd as nr

    nbytes = 65536 * 5120 * 2
    a = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        nr.nr_stream_copy(a, b)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        nr.nr_stream_copy(a, b)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return dict(kind="nr_stream_copy (16-byte streaming loads/stores, one pass)",
                bytes_per_launch=2 * nbytes, ms_per_launch=round(ms, 5),
                gbs=round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                frac_of_peak=round(2 * nbytes / (ms * 1e-3) / 1e9 / PEAK_GBS, 4))


def mix_ceilings(dev, reps=10, nbytes=65536 * 5120 * 2):
    """Practical ceilings of the three read/write mixes of the path, over
    operands of nbytes each (by default one long-sequence activation,
    65536 x 5120 bf16): one stream read and one written (copy: the forwards
    and RoPE), two read and one written (the backwards), two read and none
    written."""
    import torch

    import rmsnorm_layernorm_fwd_amd as nr

    a = torch.full((nbytes // 4,), 0x01020304, dtype=torch.int32, device=dev)
    b = torch.full_like(a, 0x10203040)
    c = torch.empty_like(a)
    probes = {"1R1W": (lambda: nr.nr_stream_copy(a, c), 2 * nbytes),
              "2R1W": (lambda: nr.nr_stream_mix(a, b, c, True), 3 * nbytes),
              "2R0W": (lambda: nr.nr_stream_mix(a, b, c, False), 2 * nbytes)}
    out = {}
    for name, (fn, moved) in probes.items():
        ms = time_fns([fn], reps)
        out[name] = dict(bytes_per_launch=moved, ms_per_launch=round(ms, 5),
                         gbs=round(moved / (ms * 1e-3) / 1e9, 1),
                         frac_of_peak=round(moved / (ms * 1e-3) / 1e9 / PEAK_GBS, 4))
    del a, b, c
    return out


def op_mix(label):
    """The read/write mix of an operation: backwards read two streams and
    write one; forwards and RoPE read one and write one."""
    return "2R1W" if label.endswith("_bwd") else "1R1W"


def cold_op_times(ops, rounds, dev):
    """Each operation timed alone with the caches cold: before every round a
    1 GiB scratch buffer is written and then read back (untimed), which
    evicts the 256 MB Infinity Cache and the L2s and leaves them holding
    clean, unrelated lines (after the write alone, the timed call would also
    pay for writing the scratch buffer's dirty lines back); then HIP events
    bracket the one call."""
    import statistics

    import torch

    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    res = {}
    for label, kname, fn, b in ops:
        ev = []
        for r in range(rounds):
            flush.fill_(r & 0x7F)
            flush.sum(dtype=torch.int64)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        t = [e0.elapsed_time(e1) for e0, e1 in ev]
        mean = statistics.fmean(t)
        res[label] = dict(kernel=kname, ms_mean=round(mean, 5),
                          ms_std=round(statistics.pstdev(t), 5), ms_min=round(min(t), 5),
                          gbs=round(b / (mean * 1e-3) / 1e9, 1),
                          frac_of_peak=round(b / (mean * 1e-3) / 1e9 / PEAK_GBS, 4))
    del flush
    return res


def warm_up(ops, warmup):
    """W warm-up steps, continued (untimed) until at least 0.5 s of steps
    have run: short steps otherwise start timing before the GPU's clocks
    have settled (the first ~20 fused-backward launches on a fresh process
    ran ~15% slower).  Returns the number of steps run."""
    import torch

    t0, done = time.perf_counter(), 0
    while done < warmup or time.perf_counter() - t0 < 0.5:
        for _, _, fn, _ in ops:
            fn()
        done += 1
        if done >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return done


def time_steps(ops, steps, warmup, only=None):
    """Warm-up (warm_up), then exactly `steps` steps timed with HIP events on
    the launch stream.  An event pair brackets every operation, or, with
    `only`, just the launches of that kernel (each pair costs a few
    microseconds of queue time, so the headline steps carry only the pairs
    the roofline needs).  Returns (warm-up steps run, ms per step, figures
    of the bracketed operations)."""
    import torch

    stream = torch.cuda.current_stream()
    done = warm_up(ops, warmup) if warmup > 0 else 0
    timed = [only is None or kname == only for _, kname, _, _ in ops]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           if timed[i] else None for i in range(len(ops))] for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(steps):
        for i, (_, _, fn, _) in enumerate(ops):
            if timed[i]:
                ev[s][i][0].record(stream)
                fn()
                ev[s][i][1].record(stream)
            else:
                fn()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps
    per_op = {}
    for i, (label, kname, _, b) in enumerate(ops):
        if not timed[i]:
            continue
        times = [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)]
        mean = sum(times) / len(times)
        std = (sum((t - mean) ** 2 for t in times) / len(times)) ** 0.5
        per_op[label] = dict(kernel=kname, bytes=b, ms_mean=round(mean, 5), ms_std=round(std, 5),
                             ms_min=round(min(times), 5),
                             gbs=round(b / (mean * 1e-3) / 1e9, 1),
                             frac_of_peak=round(b / (mean * 1e-3) / 1e9 / PEAK_GBS, 4))
    return done, ms_per_step, per_op


def dominant_kernel(ops, per_op):
    """The kernel (one instantiation, one shape) with the largest share of
    the step's time; a backward call's two kernels (rows, column sum) count
    as one "kernel" ("a+b"), since events around the call time the pair."""
    kern = {}
    for label, kname, _, b in ops:
        k = kern.setdefault(kname, dict(launches=0, bytes=0, ms=0.0, ops=[]))
        k["launches"] += 1
        k["bytes"] += b
        k["ms"] += per_op[label]["ms_mean"]
        k["ops"].append(label)
    name = max(kern, key=lambda k: kern[k]["ms"])
    return name, kern[name]


# the other configurations the 80%-of-peak bar applies to, measured in the
# default run next to the headline workload
GATED = ("rms_gemma_3840x5120", "ln_affine_15360x5120", "rope3d_15360x40x128")


def config_summary(name, steps, warmup, cold_rounds, dev):
    """One gated configuration, timed the same way as the headline workload:
    per operation in a pass with an event pair around each, the step over
    steps run back to back, and each operation alone with the caches
    flushed."""
    import torch

    ops, desc = build_ops(name, dev)
    step_bytes = sum(b for _, _, _, b in ops)
    _, _, per_op = time_steps(ops, steps, warmup)  # per operation, an event pair around each
    _, ms, _ = time_steps(ops, steps, 0, only="")  # the step, operations back to back
    cold = cold_op_times(ops, cold_rounds, dev) if cold_rounds > 0 else None
    # the mix probes over operands of this configuration's activation size
    # (a forward or RoPE operation moves about two of them), warm like the
    # operations they are set against
    act = min(b for lab, _, _, b in ops if op_mix(lab) == "1R1W") // 2 // 4096 * 4096
    mixes = mix_ceilings(dev, nbytes=act)
    out = dict(step_bytes=step_bytes, ms_per_step=round(ms, 5),
               gbs=round(step_bytes / (ms * 1e-3) / 1e9, 1),
               frac_of_peak=round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_GBS, 4),
               mix_ceilings={k: dict(gbs=v["gbs"], bytes_per_launch=v["bytes_per_launch"])
                             for k, v in mixes.items()},
               ops={k: dict(gbs=v["gbs"], frac_of_peak=v["frac_of_peak"], ms_mean=v["ms_mean"],
                            bytes=v["bytes"],
                            frac_of_mix_ceiling=round(v["gbs"] / mixes[op_mix(k)]["gbs"], 4))
                    for k, v in per_op.items()},
               ops_cold=None if cold is None else
               {k: dict(gbs=v["gbs"], frac_of_peak=v["frac_of_peak"], ms_mean=v["ms_mean"])
                for k, v in cold.items()})
    del ops
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def copy_probe(dev):
    import torch
    nbytes = 1 << 30
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes, "launches": 5}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="longseq_65536x5120",
                    choices=["longseq_65536x5120", "longseq_fused_65536x5120", "rms_gemma_3840x5120",
                             "ln_affine_15360x5120", "ln_gelu_15360x5120", "rope3d_15360x40x128",
                             "rms_linear_65536x5120x5120", "ln_linear_65536x5120x5120"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other gated configurations (3840x5120 Gemma RMSNorm, "
                         "15360x5120 LayerNorm, 15360x40x128 3-D RoPE)")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--cold-rounds", type=int, default=10,
                    help="rounds of the per-operation cold-cache timing (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: one GPU only; --gpus {args.gpus} is not supported (the operators "
              "shard by tokens, with one all-reduce of the column gradients per backward, "
              "which multi-GPU training code does in its own gradient buckets)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_probe:
        copy_probe(dev)
        return

    ops, desc = build_ops(args.workload, dev)
    step_bytes = sum(b for _, _, _, b in ops)
    # untimed calibration: an event pair around every operation gives the
    # per-operation figures ("ops") and the dominant kernel
    done, _, per_op = time_steps(ops, args.steps, args.warmup)
    dname, dk = dominant_kernel(ops, per_op)
    # the timed region: exactly K steps, event pairs only around the
    # dominant kernel's launches (for the roofline)
    _, ms_per_step, dom_ops = time_steps(ops, args.steps, 0, only=dname)
    bpl = dk["bytes"] / dk["launches"]
    mspl = sum(v["ms_mean"] for v in dom_ops.values()) / len(dom_ops)
    achieved = bpl / (mspl * 1e-3) / 1e9
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_GBS, 4), traffic=read_traffic(dname, args.workload),
                    kernel=dname, ops=dk["ops"], bytes_per_launch=int(bpl),
                    ms_per_launch=round(mspl, 5),
                    share_of_step=round(mspl * dk["launches"] / ms_per_step, 3))
    unfused = desc.pop("unfused", None)
    if "flops_per_step" in desc:
        # a contraction: the matrix cores' bf16 dense peak bounds it
        tflops = desc["flops_per_step"] / (mspl * 1e-3) / 1e12
        roofline.update(bound="mfma", achieved=round(tflops, 1), peak=PEAK_BF16_TFLOPS,
                        unit="TFLOP/s", frac=round(tflops / PEAK_BF16_TFLOPS, 4),
                        flops_per_launch=desc["flops_per_step"])
    if unfused is not None:
        ums = time_fns(unfused["fns"])
        desc["unfused_reference"] = dict(what=unfused["what"], ms=round(ums, 5),
                                         speedup_of_fused=round(ums / mspl, 4))

    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    # outside the timed steps: the copy ceiling and the cold-cache op times
    ceiling = stream_ceiling(dev)
    mixes = mix_ceilings(dev) if roofline["bound"] == "hbm" else None
    if roofline["bound"] == "hbm":
        roofline["frac_of_ceiling"] = round(achieved / ceiling["gbs"], 4)
        roofline["frac_of_mix_ceiling"] = round(achieved / mixes[op_mix(dk["ops"][0])]["gbs"], 4)
        for label, v in per_op.items():
            v["frac_of_mix_ceiling"] = round(v["gbs"] / mixes[op_mix(label)]["gbs"], 4)
    cold = cold_op_times(ops, args.cold_rounds, dev) if args.cold_rounds > 0 else None
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_steps_run": done,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded normal draws shaped like the Helios 14B activations; no model weights)",
        "config": dict(desc, step_bytes=step_bytes, frac_of_peak=round(value / PEAK_GBS, 4),
                       frac_of_ceiling=round(value / ceiling["gbs"], 4)),
        "roofline": roofline,
        "ceiling": ceiling,
        "mix_ceilings": mixes,
        "ops": per_op,
        "ops_note": ("per-operation figures from an untimed pass of K steps with an event pair "
                     "around every operation, run just before the timed steps"),
        "ops_cold": cold,
    }
    if not args.no_configs and args.workload == "longseq_65536x5120":
        out["configs"] = {name: config_summary(name, args.steps, args.warmup, args.cold_rounds, dev)
                          for name in GATED}
    if not args.no_cpu_baseline and args.workload == "longseq_65536x5120":
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
