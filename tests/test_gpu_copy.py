"""GPU check of the measurement aid nr_stream_copy: the copy the benchmark
uses as its HBM ceiling moves every byte exactly (bit-for-bit), for sizes
that end inside a workgroup's tile and for a multi-tile one."""
import pytest
import torch

import rmsnorm_layernorm_fwd_amd as nr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 48, 16 * 1024, 16 * 1024 + 16, (1 << 20) + 4096 + 32])
def test_stream_copy_exact(nbytes):
    print(f"[case] stream copy {nbytes} bytes", flush=True)
    g = torch.Generator().manual_seed(nbytes)
    src_h = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    src = src_h.to("cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    nr.nr_stream_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    out = dst.cpu()
    assert torch.equal(out[:nbytes], src_h)
    assert int(out[nbytes:].count_nonzero()) == 0  # nothing written past the end


@pytest.mark.parametrize("nbytes", [16, 48, 16 * 1024 + 16, (1 << 20) + 4096 + 32])
def test_stream_mix_exact(nbytes):
    # the two-read probe: with write, dst = a ^ b exactly and nothing past
    # the end; without, dst is untouched (the inputs' xor has no all-ones
    # 16-byte word: a's bytes are < 128 and b's are < 64)
    print(f"[case] stream mix {nbytes} bytes", flush=True)
    g = torch.Generator().manual_seed(nbytes + 1)
    a_h = torch.randint(0, 128, (nbytes,), dtype=torch.uint8, generator=g)
    b_h = torch.randint(0, 64, (nbytes,), dtype=torch.uint8, generator=g)
    a, b = a_h.to("cuda"), b_h.to("cuda")
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    nr.nr_stream_mix(a, b, dst[:nbytes], write=False)
    torch.cuda.synchronize()
    assert int(dst.count_nonzero()) == 0
    nr.nr_stream_mix(a, b, dst[:nbytes], write=True)
    torch.cuda.synchronize()
    out = dst.cpu()
    assert torch.equal(out[:nbytes], a_h ^ b_h)
    assert int(out[nbytes:].count_nonzero()) == 0
