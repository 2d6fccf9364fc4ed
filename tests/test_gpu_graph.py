"""GPU check that the library's calls can be recorded into a HIP graph: no
call allocates, synchronises or records a memset (an empty backward writes
its zero column gradients with a kernel).  One graph holds a forward and
backward of each operator; it is replayed several times with eager work and
synchronisations in between, and every replay must reproduce the eager
results bit for bit (the kernels are deterministic)."""
import pytest
import torch

import rmsnorm_layernorm_fwd_amd as nr
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_graph_replays_match_eager():
    print("[case] graph capture: rms / ln / ln+gelu / rope / fused rms+rope / rms->linear, "
          "515x1280 bf16", flush=True)
    rows, n, h, d = 515, 1280, 10, 128
    x = workloads.normal((rows, n), 9700, torch.bfloat16).to(DEV)
    w = workloads.normal((n,), 9701, torch.bfloat16, mean=1.0, std=0.1).to(DEV)
    b = workloads.normal((n,), 9702, torch.bfloat16, std=0.1).to(DEV)
    dy = workloads.normal((rows, n), 9703, torch.bfloat16).to(DEV)
    ct, st = nr.rope_table_1d(rows, d, 0, 10000.0)
    ws = torch.empty(nr.nr_bwd_workspace_bytes(rows, n, 1), dtype=torch.uint8, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    out = dict(
        y1=torch.empty_like(x), r1=torch.empty(rows, **f32), dx1=torch.empty_like(x),
        dw1=torch.empty(n, **f32),
        y2=torch.empty_like(x), mu2=torch.empty(rows, **f32), rs2=torch.empty(rows, **f32),
        dx2=torch.empty_like(x), dg2=torch.empty(n, **f32), db2=torch.empty(n, **f32),
        y3=torch.empty_like(x), mu3=torch.empty(rows, **f32), rs3=torch.empty(rows, **f32),
        dx3=torch.empty_like(x), dg3=torch.empty(n, **f32), db3=torch.empty(n, **f32),
        q=torch.empty_like(x),
        y4=torch.empty_like(x), r4=torch.empty(rows, **f32), dx4=torch.empty_like(x),
        dw4=torch.empty(n, **f32),
        e1=torch.empty(n, **f32),
        o5=torch.empty(rows, 512, dtype=torch.bfloat16, device=DEV), r5=torch.empty(rows, **f32),
        o6=torch.empty(rows, 512, dtype=torch.bfloat16, device=DEV), r6=torch.empty(rows, **f32),
    )
    Wl = workloads.normal((512, n), 9704, torch.bfloat16, std=n ** -0.5).to(DEV)
    nr.nr_tune("gemm_tile", 2)
    try:
        wsl = torch.empty(nr.nr_rmsnorm_linear_workspace_bytes(rows, 512, n, True),
                          dtype=torch.uint8, device=DEV)
    finally:
        nr.nr_tune("gemm_tile", 0)
    empty = torch.empty((0, n), dtype=torch.bfloat16, device=DEV)
    e_r = torch.empty(0, **f32)

    def step():
        o = out
        nr.rmsnorm_fwd(x, w, 1e-6, y=o["y1"], inv_rms=o["r1"])
        nr.rmsnorm_bwd(dy, x, w, o["r1"], dx=o["dx1"], dw=o["dw1"], workspace=ws)
        nr.layernorm_fwd(x, w, b, 1e-5, y=o["y2"], mean=o["mu2"], rstd=o["rs2"])
        nr.layernorm_bwd(dy, x, w, o["mu2"], o["rs2"], dx=o["dx2"], dgamma=o["dg2"],
                         dbeta=o["db2"], workspace=ws)
        nr.layernorm_gelu_fwd(x, w, b, 1e-5, y=o["y3"], mean=o["mu3"], rstd=o["rs3"])
        nr.layernorm_gelu_bwd(dy, x, w, b, o["mu3"], o["rs3"], dx=o["dx3"], dgamma=o["dg3"],
                              dbeta=o["db3"], workspace=ws)
        o["q"].copy_(x)
        nr.rope_interleaved_apply(o["q"].view(1, rows, h, d), ct, st)
        nr.rmsnorm_rope_fwd(x, w, ct, st, d, 1, 1e-6, y=o["y4"], inv_rms=o["r4"])
        nr.rmsnorm_rope_bwd(dy, x, w, o["r4"], ct, st, d, 1, dx=o["dx4"], dw=o["dw4"],
                            workspace=ws)
        # RMSNorm -> linear on both kernels (the 256 x 256 one: statistics,
        # weight fold and GEMM, three launches)
        nr.rmsnorm_linear_fwd(x, w, Wl, out=o["o5"], inv_rms=o["r5"])
        nr.nr_tune("gemm_tile", 2)
        try:
            nr.rmsnorm_linear_fwd(x, w, Wl, out=o["o6"], inv_rms=o["r6"], workspace=wsl)
        finally:
            nr.nr_tune("gemm_tile", 0)
        # an empty batch: its column gradient (zeros) comes from a kernel
        o["e1"].fill_(7.0)
        nr.rmsnorm_bwd(empty, empty, w, e_r, dx=torch.empty_like(empty), dw=o["e1"],
                       workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in out.items()}
    assert torch.all(eager["e1"] == 0)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for v in out.values():
            v.fill_(float("nan") if v.dtype.is_floating_point else 0)  # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in out.items():
            assert torch.equal(v, eager[k]), f"replay {rep}: {k} differs from the eager result"
