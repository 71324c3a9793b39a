"""GPU check of the measurement probe (register-only bf16 MFMA loop with clock stamps)."""
import numpy as np
import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu


def test_mfma_probe_stamps_and_rate(gpu_lib):
    import torch

    blocks, iters = 512, 2000
    say("probe", blocks, iters)
    gpu_lib.probe_mfma_bf16(blocks, iters)                 # warm-up
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    clocks = gpu_lib.probe_mfma_bf16(blocks, iters)
    e1.record()
    e1.synchronize()
    c = clocks.cpu().numpy().astype(np.float64)
    assert c.shape == (blocks, 4)
    assert np.all(c[:, 2] > c[:, 0]) and np.all(c[:, 3] > c[:, 1])   # both counters advance
    mhz = np.median(100.0 * (c[:, 2] - c[:, 0]) / (c[:, 3] - c[:, 1]))
    tflops = blocks * 4 * iters * 8 * 16384 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    say("probe", {"sclk_mhz": float(mhz), "tflops": tflops})
    assert 300.0 < mhz < 3500.0                 # a shader clock, in MHz
    assert 0.0 < tflops < 2.6e3                 # never above the datasheet bf16 peak (2.5 PFLOP/s) + 4%


def test_copy_and_read_probes(gpu_lib):
    import torch

    for nbytes, blocks in ((16, 0), (4096 + 48, 0), (3 << 20, 0), (3 << 20, 7), (64 << 20, 0)):
        say("bandwidth probe", nbytes, blocks)
        g = torch.Generator(device="cuda")
        g.manual_seed(nbytes + blocks)
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4 + 8,), generator=g, dtype=torch.int32,
                            device="cuda")
        dst = torch.full_like(src, 7)
        gpu_lib.probe_copy(src, dst, nbytes, blocks)
        torch.cuda.synchronize()
        q = nbytes // 4
        assert torch.equal(dst[:q], src[:q])
        assert torch.all(dst[q:] == 7)                      # nothing past the bytes
        sink = torch.full((4,), 5, dtype=torch.int32, device="cuda")
        gpu_lib.probe_read(src, sink, nbytes, blocks, key=0x12345677)
        torch.cuda.synchronize()
        got = sink.cpu().numpy().view(np.uint32)
        assert got[0] in (5, 0x12345677) and np.all(got[1:] == 5)
