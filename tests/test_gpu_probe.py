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
