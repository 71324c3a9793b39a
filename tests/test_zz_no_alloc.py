"""GPU check of qgemm_int4_noalloc, the int4 entry point that allocates nothing
(its workspace is the library's static per-GPU scratch), called through the C
ABI with raw pointers: its output equals qgemm_int4's with a workspace, bit for
bit, and passes the oracle's rule; two calls in a row, the second smaller, for
each path that uses the workspace (k split of the small-M kernel, prepared
activations and k split of the MFMA tiles)."""
import ctypes

import numpy as np
import pytest

import oracle
from qgemm_inputs import int4_inputs

from gpu_helpers import host_u16, say, upload_int4

pytestmark = pytest.mark.gpu

QG_ERR_SCRATCH = 8

# (first, second) shapes (m, k, n); the second call of each pair is smaller
PAIRS = [
    ((8, 16384, 520), (8, 8192, 264)),       # small-M k split (counters + partials), then a smaller split
    ((1, 20480, 776), (1, 16384, 264)),      # GEMV k split, then a smaller one
    ((130, 8192, 776), (80, 4096, 264)),     # MFMA tiles: prepared activations + k split, then smaller
    ((512, 5120, 2048), (65, 2048, 1040)),   # MFMA tiles with preparation and split, then smaller
    ((96, 5120, 1024), (17, 2048, 520)),     # then the two-row-tile small-M kernel (no workspace)
]


def call_noalloc(qg, t, y):
    import torch

    lib = qg.load()
    m, k = t["x"].shape
    n = t["qweight"].shape[1]
    st = lib.qgemm_int4_noalloc(t["x"].data_ptr(), k, t["qweight"].data_ptr(), t["scales"].data_ptr(),
                                t["qzeros"].data_ptr(), y.data_ptr(), n, m, n, k, 128,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("pair", PAIRS, ids=["%dx%dx%d-then-%dx%dx%d" % (a + b) for a, b in PAIRS])
def test_noalloc_matches_the_workspace_entry_point(gpu_lib, pair):
    import torch

    for i, (m, k, n) in enumerate(pair):
        desc = gpu_lib.describe_int4(m, n, k)
        say("noalloc", i, m, k, n, desc, "workspace", gpu_lib.workspace_size(m, n, k))
        d = int4_inputs(m, k, n, seed=7000 + 10 * i + m)
        t = upload_int4(d)
        y_ws = gpu_lib.qgemm_int4(t["x"], t["qweight"], t["scales"], t["qzeros"])
        y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda")
        assert call_noalloc(gpu_lib, t, y) == 0
        torch.cuda.synchronize()
        a, b = host_u16(y), host_u16(y_ws)
        assert np.array_equal(a, b), (m, k, n, int(np.sum(a != b)))
        ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
        rep = oracle.compare(a, ref, "bf16")
        say("noalloc", i, rep)
        assert rep["rejected"] == 0 and rep["nonfinite"] == 0, rep
        # the counters were left at zero: the same call again gives the same bits
        y2 = torch.empty_like(y)
        assert call_noalloc(gpu_lib, t, y2) == 0
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(y2), a)


def test_noalloc_rejects_a_problem_beyond_the_scratch(gpu_lib):
    import torch

    m, k, n = 2048, 25600, 64
    assert gpu_lib.workspace_size(m, n, k) > 32 << 20
    t = {"x": torch.zeros((m, k), dtype=torch.bfloat16, device="cuda"),
         "qweight": torch.zeros((k // 8, n), dtype=torch.int32, device="cuda"),
         "scales": torch.zeros((k // 128, n), dtype=torch.float16, device="cuda"),
         "qzeros": torch.zeros((k // 128, n // 8), dtype=torch.int32, device="cuda")}
    y = torch.full((m, n), 3.0, dtype=torch.bfloat16, device="cuda")
    assert call_noalloc(gpu_lib, t, y) == QG_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)          # nothing was launched
