"""The Python binding's argument checks: tensors the C ABI cannot take are
refused with ValueError before any call into the library (nothing is
launched, the outputs keep their contents)."""
import pytest
import torch

import oracle
import rmsnorm_layernorm_fwd_amd as nr
from tolerance import check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(rows=8, n=256, dtype=torch.bfloat16):
    x = torch.randn(rows, n, device=DEV).to(dtype)
    w = torch.ones(n, device=DEV, dtype=dtype)
    return x, w


def test_host_tensor_refused():
    print("[case] binding: host tensors", flush=True)
    x, w = _inputs()
    with pytest.raises(ValueError, match="GPU tensor"):
        nr.rmsnorm_fwd(x, w.cpu())
    with pytest.raises(ValueError, match="GPU tensor"):
        nr.rmsnorm_fwd(x.cpu(), w)


def test_dtype_shape_and_layout_refused():
    print("[case] binding: dtype, shape, layout", flush=True)
    x, w = _inputs()
    y = torch.full_like(x, 7.0)
    with pytest.raises(ValueError, match="must be torch.bfloat16"):
        nr.rmsnorm_fwd(x, w.float(), y=y)
    with pytest.raises(ValueError, match="shape"):
        nr.rmsnorm_fwd(x, w[:128].contiguous(), y=y)
    with pytest.raises(ValueError, match="contiguous"):
        nr.rmsnorm_fwd(x, torch.ones(512, device=DEV, dtype=x.dtype)[::2], y=y)
    with pytest.raises(ValueError, match="shape"):
        nr.layernorm_fwd(x, w, w, y=torch.empty(8, 128, device=DEV, dtype=x.dtype))
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)  # nothing ran


def test_workspace_on_host_refused():
    print("[case] binding: host workspace", flush=True)
    x, w = _inputs()
    _, r = nr.rmsnorm_fwd(x, w)
    ws = torch.empty(nr.nr_bwd_workspace_bytes(8, 256, 0), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        nr.rmsnorm_bwd(torch.ones_like(x), x, w, r, workspace=ws)


def test_device_check_compares_devices():
    # the binding checks every tensor against the first one's device; on a
    # one-GPU machine the rule is exercised directly
    print("[case] binding: device rule", flush=True)
    x, _ = _inputs()
    nr._dev("x", x, device=x.device)  # same device: accepted
    with pytest.raises(ValueError, match="must be on"):
        nr._dev("x", x, device=torch.device("cuda", x.device.index + 1))


def test_calls_run_on_the_tensors_device_with_its_stream():
    # a side stream made current: the call is ordered on it (the result is
    # complete once that stream is synchronised)
    print("[case] binding: current stream", flush=True)
    x, w = _inputs(rows=4096, n=1024)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        y, r = nr.rmsnorm_fwd(x, w)
    s.synchronize()
    # once the side stream is synchronised the result is complete: it is
    # held to the oracle's fp64 values within the usual one-ulp bound
    ry, rr = oracle.rmsnorm_fwd(x.cpu(), w.cpu(), 1e-6)
    check("side stream y", y.cpu(), ry, "bf16")
    check("side stream inv_rms", r.cpu(), rr, "stat", s=0.0)


def test_overlapping_buffers_refused_by_the_library():
    # buffers the binding accepts (right dtype, shape, device) but that share
    # bytes with another operand: the library refuses them (NR_ERR_ALIAS)
    # before queuing anything, and the outputs keep their contents
    print("[case] binding: overlapping buffers", flush=True)
    x, w = _inputs(rows=8, n=256, dtype=torch.float32)
    dy = torch.randn_like(x)
    y, r = nr.rmsnorm_fwd(x, w)
    torch.cuda.synchronize()
    # the column gradient inside dy's storage
    dw_view = dy.view(-1)[:256]
    before = dy.clone()
    with pytest.raises(nr.NormRopeError):
        nr.rmsnorm_bwd(dy, x, w, r, dw=dw_view)
    torch.cuda.synchronize()
    assert torch.equal(dy, before)
    # the row statistics inside the output of the forward
    y2 = torch.full_like(x, 7.0)
    with pytest.raises(nr.NormRopeError):
        nr.rmsnorm_fwd(x, w, y=y2, inv_rms=y2.view(-1)[:8])
    torch.cuda.synchronize()
    assert torch.all(y2 == 7.0)
    # RoPE tables inside the tensor they rotate
    q = torch.randn(1, 4, 2, 8, device=DEV)
    qc = q.clone()
    with pytest.raises(nr.NormRopeError):
        nr.rope_interleaved_apply(q, q.view(-1)[:16].view(4, 4), q.view(-1)[16:32].view(4, 4))
    torch.cuda.synchronize()
    assert torch.equal(q, qc)
