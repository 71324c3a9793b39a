"""GPU parity of the int4 GPTQ paths against the CPU oracle (through the C ABI).

The reference is the C++ oracle (oracle/qgemm_oracle_cpu.cpp: dequantise to
fp32, accumulate in fp64) for the dequantised weights, every path at small
shapes and the sampled full sizes; the numpy oracle, pinned separately, is the
reference of the remaining cases.  Bar: dequantised weights bit-exact; products accepted element by element by
the oracle's rule (|err| <= 2e-3 + 2e-3 |ref| or a faithful bf16 rounding),
with zero rejections, no non-finite values and rms_rel at the bf16 rounding
floor.  One-hot rows and blocked sums are exact and compared bitwise.
"""
import numpy as np
import pytest

import oracle
from oracle import cpu as cpp_oracle
from qgemm_inputs import f32_to_bf16_bits, int4_cases, int4_inputs

from gpu_helpers import dev, host_u16, host_u32, sample_indices, say, upload_int4

pytestmark = pytest.mark.gpu

RMS_GATE = 2.5e-3


def run(qg, t, path="auto", out=None, workspace=None):
    import torch

    y = qg.qgemm_int4(t["x"], t["qweight"], t["scales"], t["qzeros"], out=out, path=path,
                      workspace=workspace)
    torch.cuda.synchronize()
    return y


def assert_accepted(y_bits, ref, what):
    rep = oracle.compare(y_bits, ref, "bf16")
    say(what, rep)
    assert rep["nonfinite"] == 0, (what, rep)
    assert rep["rejected"] == 0, (what, rep)
    if np.sqrt(np.mean(ref * ref)) > 0.05:
        assert rep["rms_rel"] < RMS_GATE, (what, rep)


# ----------------------------------------------------------------------------
# dequant: bit-exact
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("k,n", [(128, 8), (1152, 776), (4096, 4096), (896, 4864)])
def test_dequant_bit_exact(gpu_lib, k, n):
    say("dequant", k, n)
    d = int4_inputs(1, k, n, seed=100 + k + n)
    t = upload_int4(d)
    w = gpu_lib.qgemm_int4_dequant(t["qweight"], t["scales"], t["qzeros"])
    ref = cpp_oracle.dequant(d["qweight"], d["scales"], d["qzeros"], k, n)
    assert np.array_equal(host_u32(w), ref.view(np.uint32))
    assert np.array_equal(ref, oracle.dequant(d["qweight"], d["scales"], d["qzeros"], k, n))


# ----------------------------------------------------------------------------
# every path on shapes the oracle finishes quickly: several tiles + ragged tails
# ----------------------------------------------------------------------------
SMALL_SHAPES = [(128, 8), (1152, 776), (2048, 1040), (128, 12296), (256, 24584)]
PATH_MS = {
    "gemv": [1],
    "fused": [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16],
    "mfma": [1, 16, 17, 33, 130, 257],
    "mfma_nows": [17, 33, 130, 257],     # no workspace: the MFMA tiles without the preparation pass
    "auto": [1, 6, 16, 17, 24, 32, 33, 40, 48, 64, 200],   # 17..64: two to four MFMA row tiles
}


@pytest.mark.parametrize("k,n", SMALL_SHAPES)
@pytest.mark.parametrize("path", ["gemv", "fused", "mfma", "mfma_nows", "auto"])
def test_paths_match_oracle(gpu_lib, path, k, n):
    p, ws = ("mfma", False) if path == "mfma_nows" else (path, None)
    for m in PATH_MS[path]:
        if m * n * k > 2 ** 31:
            continue
        say("path", path, "m", m, "k", k, "n", n)
        d = int4_inputs(m, k, n, seed=7 * m + k + n)
        y = run(gpu_lib, upload_int4(d), p, workspace=ws)
        ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
        assert_accepted(host_u16(y), ref, (path, m, k, n))


# ----------------------------------------------------------------------------
# exact cases, compared bitwise
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("path", ["gemv", "fused", "mfma"])
def test_one_hot_rows_are_exact(gpu_lib, path):
    k, n = 1152, 776
    rows = [200] if path == "gemv" else [0, 7, 8, 127, 128, 1151]
    d = int4_inputs(1, k, n, seed=31)
    x = np.zeros((len(rows), k), dtype=np.uint16)
    for r, i in enumerate(rows):
        x[r, i] = 0x3F80
    d["x"] = x
    say("one-hot", path, rows)
    y = host_u16(run(gpu_lib, upload_int4(d), path))
    w = oracle.dequant(d["qweight"], d["scales"], d["qzeros"], k, n)
    expect = f32_to_bf16_bits(w[rows, :])
    assert np.array_equal(y, expect)


@pytest.mark.parametrize("path", ["gemv", "fused", "mfma"])
def test_blocked_sum_is_exact(gpu_lib, path):
    # X = 1 on group 2 only and q - z = 5: Y = bf16(640 * s[2][j]) exactly
    k, n = 640, 264
    m = 1 if path == "gemv" else 3
    d = int4_inputs(m, k, n, seed=32)
    d["x"] = np.zeros((m, k), dtype=np.uint16)
    d["x"][:, 256:384] = 0x3F80
    d["qweight"] = np.full((k // 8, n), 0x77777777, dtype=np.uint32)
    d["qzeros"] = np.full((k // 128, n // 8), 0x22222222, dtype=np.uint32)
    say("blocked", path)
    y = host_u16(run(gpu_lib, upload_int4(d), path))
    s2 = oracle.fp16_value(d["scales"][2])
    assert np.array_equal(y, np.repeat(f32_to_bf16_bits(640.0 * s2)[None, :], m, axis=0))


@pytest.mark.parametrize("path", ["gemv", "fused", "mfma"])
def test_codes_equal_zeros_give_zero(gpu_lib, path):
    # w = 0 everywhere.  The kernels subtract the zero point through the group sum
    # of the activations, so the result is zero up to fp32 rounding of that
    # cancellation (far below the acceptance bound), not bitwise.
    k, n = 1024, 136
    m = 1 if path == "gemv" else 5
    d = int4_inputs(m, k, n, seed=33)
    z = oracle.unpack_qzeros(d["qzeros"], k // 128, n)
    zrow = z[np.arange(k // 8) // 16, :].astype(np.uint32)
    d["qweight"] = (zrow * np.uint32(0x11111111)).astype(np.uint32)
    assert np.all(oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n) == 0)
    say("q==z", path)
    y = oracle.bf16_value(host_u16(run(gpu_lib, upload_int4(d), path)))
    assert np.max(np.abs(y)) < 1e-4


@pytest.mark.parametrize("m,paths", [(5, ["fused", "mfma"]), (1, ["gemv", "fused"]), (16, ["fused"])])
def test_strided_x_and_y_with_guard_bands(gpu_lib, m, paths):
    import torch

    k, n = 1024, 520
    d = int4_inputs(m, k, n, seed=34 + m)
    t = upload_int4(d)
    xs = torch.zeros((m, k + 64), dtype=torch.bfloat16, device="cuda")
    xs[:, :k] = t["x"]
    t["x"] = xs[:, :k]
    for path in paths:
        big = torch.full((m + 2, n + 24), -384.0, dtype=torch.bfloat16, device="cuda")
        out = big[1:m + 1, 8:8 + n]
        say("strided", path)
        run(gpu_lib, t, path, out=out)
        ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
        assert_accepted(host_u16(out), ref, ("strided", path))
        b = big.float().cpu().numpy()
        b[1:m + 1, 8:8 + n] = -384.0
        assert np.all(b == -384.0), "write outside the output view"


@pytest.mark.parametrize("m,k,n", [(24, 1024, 520), (32, 16384, 264), (17, 128, 8), (32, 128, 8),
                                   (40, 2048, 1040), (48, 16384, 264), (56, 1024, 520), (64, 16384, 264),
                                   (33, 128, 8), (64, 128, 8)])
def test_row_tiles_strided_guarded_and_tiny(gpu_lib, m, k, n):
    # the small-M kernel with two to four MFMA row tiles (automatic path): strided
    # X and Y inside guard bands, a k split (k = 16384), and the smallest k and n
    import torch

    d = int4_inputs(m, k, n, seed=35 + m + k)
    t = upload_int4(d)
    xs = torch.zeros((m, k + 64), dtype=torch.bfloat16, device="cuda")
    xs[:, :k] = t["x"]
    t["x"] = xs[:, :k]
    big = torch.full((m + 2, n + 24), -384.0, dtype=torch.bfloat16, device="cuda")
    out = big[1:m + 1, 8:8 + n]
    say("row tiles strided", m, k, n, gpu_lib.describe_int4(m, n, k))
    assert gpu_lib.describe_int4(m, n, k).startswith("skinny_int4_kernel<%d,mfma," % m)
    run(gpu_lib, t, "auto", out=out)
    ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    assert_accepted(host_u16(out), ref, ("row tiles strided", m, k, n))
    b = big.float().cpu().numpy()
    b[1:m + 1, 8:8 + n] = -384.0
    assert np.all(b == -384.0), "write outside the output view"


def test_k_zero_writes_zeros_and_m_zero_is_noop(gpu_lib):
    import torch

    t = {"x": torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda"),
         "qweight": torch.zeros((0, 64), dtype=torch.int32, device="cuda"),
         "scales": torch.zeros((0, 64), dtype=torch.float16, device="cuda"),
         "qzeros": torch.zeros((0, 8), dtype=torch.int32, device="cuda")}
    out = torch.full((3, 64), 5.0, dtype=torch.bfloat16, device="cuda")
    run(gpu_lib, t, out=out)
    assert torch.all(out == 0)
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    t0 = dict(t, x=torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda"))
    run(gpu_lib, t0, out=e)


SPLIT_SHAPES = [(16384, 520), (20480, 776)]       # long k, few strips: the k split is on


@pytest.mark.parametrize("k,n", SPLIT_SHAPES)
@pytest.mark.parametrize("path,m", [("gemv", 1), ("fused", 1), ("fused", 8), ("fused", 16)])
def test_split_k_with_and_without_workspace(gpu_lib, path, m, k, n):
    d = int4_inputs(m, k, n, seed=36 + m + n)
    t = upload_int4(d)
    ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    for ws in (None, False):
        say("split", path, m, k, n, "ws" if ws is None else "no-ws",
            gpu_lib.describe_int4(m, n, k, path, None if ws is None else 0))
        y = run(gpu_lib, t, path, workspace=ws)
        assert_accepted(host_u16(y), ref, ("split", path, m, k, n, ws))


# MFMA tiles with a k split (few tiles, long k): partial tiles, per-tile tickets and
# the ordered reduction by the last slice; the first shapes leave ragged tiles
MFMA_SPLIT_SHAPES = [(33, 4096, 520), (130, 8192, 776), (17, 16384, 264), (64, 6144, 1040)]


@pytest.mark.parametrize("m,k,n", MFMA_SPLIT_SHAPES)
def test_mfma_split_k_matches_oracle(gpu_lib, m, k, n):
    desc = gpu_lib.describe_int4(m, n, k, "mfma")
    say("mfma-split", m, k, n, desc)
    assert "ksplit=1 " not in desc + " "
    d = int4_inputs(m, k, n, seed=50 + m + n)
    t = upload_int4(d)
    ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    y1 = run(gpu_lib, t, "mfma")
    assert_accepted(host_u16(y1), ref, ("mfma-split", m, k, n))
    y2 = run(gpu_lib, t, "mfma")            # the tickets were reset: same result again
    assert np.array_equal(host_u16(y1), host_u16(y2))


# the k split under both exchange orders: the small-M kernel's strips (16 slices), the
# GEMV, and the MFMA tiles (a ticket per tile); acquire-release tickets give the same
# sums, bit for bit
@pytest.mark.parametrize("path,m,k,n", [("fused", 8, 16384, 520), ("gemv", 1, 20480, 776),
                                        ("mfma", 130, 8192, 776), ("mfma", 17, 16384, 264)])
def test_split_orders_agree(gpu_lib, path, m, k, n):
    desc = gpu_lib.describe_int4(m, n, k, path)
    say("split-order", path, m, k, n, desc)
    assert "ksplit=1 " not in desc + " "
    d = int4_inputs(m, k, n, seed=50 + m)
    t = upload_int4(d)
    ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    assert gpu_lib.split_order() == "hw"
    y_hw = host_u16(run(gpu_lib, t, path))
    try:
        gpu_lib.set_split_order("acq_rel")
        y_ar = host_u16(run(gpu_lib, t, path))
        y_ar2 = host_u16(run(gpu_lib, t, path))      # the tickets were reset under this order too
    finally:
        gpu_lib.set_split_order("hw")
    assert_accepted(y_ar, ref, ("split-order", path, m, k, n))
    assert np.array_equal(y_ar, y_hw) and np.array_equal(y_ar2, y_hw)


# 128-column strips (m <= 16, k split anyway, long slices): ragged last strip (4104 = 32 x 128
# + 8 columns), 7 slices of 23 groups; every output against the C++ oracle, the same bits
# again (tickets reset) and under acquire-release tickets; without a workspace the plan
# falls back to 64-column strips without a split
@pytest.mark.parametrize("path,m,k,n", [("auto", 3, 20480, 4104), ("auto", 16, 20480, 4104),
                                        ("fused", 1, 20480, 4104)])
def test_wide_strips_match_oracle(gpu_lib, path, m, k, n):
    desc = gpu_lib.describe_int4(m, n, k, path)
    say("wide-strips", path, m, k, n, desc)
    assert ",mfma,8>" in desc and "ksplit=1 " not in desc + " "
    d = int4_inputs(m, k, n, seed=1700 + m)
    t = upload_int4(d)
    ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    y1 = host_u16(run(gpu_lib, t, path))
    assert_accepted(y1, ref, ("wide-strips", path, m, k, n))
    assert np.array_equal(y1, host_u16(run(gpu_lib, t, path)))
    try:
        gpu_lib.set_split_order("acq_rel")
        y_ar = host_u16(run(gpu_lib, t, path))
    finally:
        gpu_lib.set_split_order("hw")
    assert np.array_equal(y1, y_ar)
    assert ",mfma,8>" not in gpu_lib.describe_int4(m, n, k, path, 0)
    y0 = host_u16(run(gpu_lib, t, path, workspace=False))
    assert_accepted(y0, ref, ("wide-strips no-ws", path, m, k, n))


# 128-column strips without a split (more 64-column strips than two per CU hold in one
# pass, 193 of 128 columns with a ragged last one): every output against the C++ oracle
@pytest.mark.parametrize("path,m,k,n", [("auto", 5, 4096, 24584), ("auto", 16, 6144, 24584),
                                        ("fused", 1, 4096, 24584)])
def test_wide_strips_unsplit_match_oracle(gpu_lib, path, m, k, n):
    desc = gpu_lib.describe_int4(m, n, k, path)
    say("wide-strips-unsplit", path, m, k, n, desc)
    assert ",mfma,8> grid=" in desc and "ksplit=1 " in desc + " "
    d = int4_inputs(m, k, n, seed=1750 + m)
    t = upload_int4(d)
    ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    y = host_u16(run(gpu_lib, t, path))
    assert_accepted(y, ref, ("wide-strips-unsplit", path, m, k, n))


def test_gemv_long_k_without_workspace(gpu_lib):
    # 600 groups on one 16-column strip, no k split: each wave walks a long chain
    m, k, n = 1, 76800, 16
    desc = gpu_lib.describe_int4(m, n, k, "gemv", 0)
    say("long-k", desc)
    assert "dot" in desc and "ksplit=1" in desc
    d = int4_inputs(m, k, n, seed=39)
    y = run(gpu_lib, upload_int4(d), "gemv", workspace=False)
    ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    assert_accepted(host_u16(y), ref, ("long-k", m, k, n))


def test_shared_workspace_across_shapes_and_counters_reset(gpu_lib):
    import torch

    ws = torch.zeros(8 << 20, dtype=torch.uint8, device="cuda")
    # includes m > 16 calls, whose preparation pass writes past the counters
    shapes = [(8, 16384, 520), (1, 20480, 776), (40, 2048, 520), (15, 1152, 776), (16, 16384, 1040),
              (130, 1152, 776), (3, 896, 4864), (8, 16384, 520)]
    for i, (m, k, n) in enumerate(shapes):
        say("shared-ws", m, k, n, gpu_lib.describe_int4(m, n, k, workspace_bytes=ws.numel()))
        d = int4_inputs(m, k, n, seed=40 + i)
        y = run(gpu_lib, upload_int4(d), workspace=ws)
        ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
        assert_accepted(host_u16(y), ref, ("shared-ws", m, k, n))
        # the split's counters (the first 64 KiB) are back at zero
        assert int(torch.count_nonzero(ws[:65536])) == 0


def test_first_split_call_on_a_side_stream(gpu_lib):
    # the binding's cached workspace for a stream it has not seen is created and
    # zero-filled on that stream, ordered before the kernels that read its
    # counters; the first call on a fresh, non-current stream takes the k split
    import torch

    m, k, n = 8, 16384, 520
    assert "ksplit=1 " not in gpu_lib.describe_int4(m, n, k) + " "
    d = int4_inputs(m, k, n, seed=34)
    t = upload_int4(d)
    ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    assert side.cuda_stream != torch.cuda.current_stream().cuda_stream
    outs = [torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    for o in outs:
        gpu_lib.qgemm_int4(t["x"], t["qweight"], t["scales"], t["qzeros"], out=o, stream=side)
    side.synchronize()
    for o in outs:
        assert_accepted(host_u16(o), ref, ("side-stream", m, k, n))
    # also through a raw stream handle (the workspace of that stream is reused)
    o = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    gpu_lib.qgemm_int4(t["x"], t["qweight"], t["scales"], t["qzeros"], out=o, stream=side.cuda_stream)
    side.synchronize()
    assert np.array_equal(host_u16(o), host_u16(outs[0]))


def test_deterministic(gpu_lib):
    m, k, n = 8, 2048, 1040
    d = int4_inputs(m, k, n, seed=35)
    t = upload_int4(d)
    for path in ["fused", "mfma"]:
        a = host_u16(run(gpu_lib, t, path))
        b = host_u16(run(gpu_lib, t, path))
        assert np.array_equal(a, b)
    m1 = int4_inputs(1, k, n, seed=37)
    t1 = upload_int4(m1)
    assert np.array_equal(host_u16(run(gpu_lib, t1, "gemv")), host_u16(run(gpu_lib, t1, "gemv")))
    # with the k split on, partials are added in k order: still deterministic
    d2 = int4_inputs(8, 16384, 520, seed=38)
    t2 = upload_int4(d2)
    assert np.array_equal(host_u16(run(gpu_lib, t2, "fused")), host_u16(run(gpu_lib, t2, "fused")))


# ----------------------------------------------------------------------------
# full workload sizes, the launch configuration the benchmark times (auto path),
# checked on sampled outputs the oracle computes one by one
# ----------------------------------------------------------------------------
FULL = [(c, case) for c in (0, 1, 2, 4) for case in int4_cases(c)]
# 17..32 tokens at workload sizes: two row tiles with a k split (25600 x 5120), at n >= 20480 (m <= 24,
# and m = 32 in two passes), and the MFMA tiles beyond two passes (m = 32, 8192 x 28672)
FULL += [(2, ("row-tiles", 20, 25600, 5120, 2020)), (2, ("row-tiles", 24, 5120, 25600, 2024)),
         (2, ("row-tiles", 32, 5120, 25600, 2032)), (1, ("row-tiles", 17, 4096, 4096, 1017)),
         (3, ("row-tiles", 32, 8192, 28672, 3032))]
# 257..383 strips: 8-wave workgroups, two per CU (2048 x 5632: 352 strips)
FULL += [(1, ("strips", 8, 2048, 5632, 1108)), (1, ("strips", 1, 2048, 5632, 1101))]
# the LDS-staged kernel over the whole k where the register-staged plan splits it:
# 32-column strips with 4 groups per wave (16 and 14 waves), and the GEMV's 16-column strips
FULL += [(1, ("whole-k", 16, 8192, 8192, 1116)), (1, ("whole-k", 8, 7168, 8192, 1118)),
         (1, ("whole-k", 1, 8192, 5632, 1119))]
# 33..64 tokens: three and four row tiles in one pass over the CUs (4096 x 4096, 2048 x 8192)
FULL += [(1, ("row-tiles", 33, 4096, 4096, 1033)), (1, ("row-tiles", 64, 4096, 4096, 1064)),
         (1, ("row-tiles", 48, 2048, 8192, 1048)), (2, ("row-tiles", 40, 14336, 4096, 2040))]   # two passes, k split


@pytest.mark.parametrize("cfg,case", FULL, ids=["c%d-m%d-k%d-n%d" % (c, x[1], x[2], x[3]) for c, x in FULL])
def test_full_size_sampled(gpu_lib, cfg, case):
    _, m, k, n, seed = case
    say("full", cfg, m, k, n)
    d = int4_inputs(m, k, n, seed=seed)
    y = host_u16(run(gpu_lib, upload_int4(d)))
    rows = sample_indices(m, 24, seed)
    cols = sample_indices(n, 160, seed + 1)
    ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n, rows=rows, cols=cols)
    assert_accepted(y[np.ix_(rows, cols)], ref, ("full", cfg, m, k, n))


# ----------------------------------------------------------------------------
# weights without a zero point (qzeros NULL: w = q * s), every path
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("k,n", [(128, 8), (1152, 776)])
def test_dequant_without_zero_point_bit_exact(gpu_lib, k, n):
    say("dequant-nozero", k, n)
    d = int4_inputs(1, k, n, seed=300 + k + n)
    t = upload_int4(d)
    w = gpu_lib.qgemm_int4_dequant(t["qweight"], t["scales"], None)
    ref = cpp_oracle.dequant(d["qweight"], d["scales"], None, k, n)
    assert np.array_equal(host_u32(w), ref.view(np.uint32))


NOZERO_CASES = [("gemv", 1, 1152, 776), ("fused", 2, 2048, 1040), ("fused", 8, 1152, 776),
                ("fused", 15, 2048, 1040), ("fused", 16, 1152, 776), ("mfma", 17, 2048, 1040),
                ("mfma", 130, 1152, 776), ("mfma_nows", 33, 2048, 1040),
                ("gemv", 1, 16384, 520), ("fused", 8, 16384, 520), ("mfma", 33, 4096, 520),
                ("auto", 24, 16384, 520), ("auto", 31, 2048, 1040),   # two row tiles (k split / none)
                ("auto", 48, 2048, 1040), ("auto", 64, 16384, 264),   # three / four row tiles
                ("fused", 4, 16384, 520)]   # MFMA strips with idle waves (16 waves, 8 groups per k slice)


@pytest.mark.parametrize("path,m,k,n", NOZERO_CASES)
def test_paths_without_zero_point_match_oracle(gpu_lib, path, m, k, n):
    p, ws = ("mfma", False) if path == "mfma_nows" else (path, None)
    say("nozero", path, m, k, n, gpu_lib.describe_int4(m, n, k, p, None if ws is None else 0))
    d = int4_inputs(m, k, n, seed=400 + m + k + n)
    t = dict(upload_int4(d), qzeros=None)
    y = run(gpu_lib, t, p, workspace=ws)
    ref = cpp_oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], None, m, k, n)
    assert_accepted(host_u16(y), ref, ("nozero", path, m, k, n))


@pytest.mark.parametrize("m,k,n", [(1, 4096, 4096), (15, 2048, 8192), (512, 5120, 25600)])
def test_full_size_without_zero_point_sampled(gpu_lib, m, k, n):
    say("nozero-full", m, k, n)
    d = int4_inputs(m, k, n, seed=500 + m)
    y = host_u16(run(gpu_lib, dict(upload_int4(d), qzeros=None)))
    rows = sample_indices(m, 24, m)
    cols = sample_indices(n, 160, m + 1)
    ref = oracle.qgemm_int4_at(d["x"], d["qweight"], d["scales"], None, k, n, rows, cols)
    assert_accepted(y[np.ix_(rows, cols)], ref, ("nozero-full", m, k, n))


# ----------------------------------------------------------------------------
# LoRA add in the epilogue (qgemm_int4_lora): every path, with and without the
# k split / preparation, ranks 16 and 5, full sizes sampled
# ----------------------------------------------------------------------------
from qgemm_inputs import lora_inputs  # noqa: E402


def upload_lora(l):
    import torch

    return dev(l["lora_a"], torch.bfloat16), dev(l["lora_b"], torch.bfloat16)


LORA_CASES = [("gemv", 1, 1152, 776, 16), ("fused", 2, 2048, 1040, 16), ("fused", 8, 1152, 776, 5),
              ("fused", 15, 2048, 1040, 16), ("fused", 16, 1152, 776, 16), ("mfma", 17, 2048, 1040, 16),
              ("mfma", 130, 1152, 776, 5), ("mfma", 257, 2048, 1040, 16),
              ("gemv", 1, 16384, 520, 16), ("fused", 8, 16384, 520, 16), ("mfma", 33, 4096, 520, 16),
              ("auto", 24, 2048, 1040, 16), ("auto", 32, 16384, 520, 5), ("auto", 31, 1152, 776, 1),   # two row tiles
              ("auto", 40, 2048, 1040, 16), ("auto", 64, 16384, 264, 3),   # three / four row tiles
              ("fused", 4, 16384, 520, 16),   # idle waves
              # U accumulated in the product's launch: the LDS-staged kernel with the
              # activations in registers (two workgroups per CU) and with 64-column strips
              ("fused", 15, 2048, 5632, 16), ("auto", 1, 4096, 14336, 7), ("fused", 3, 4096, 14336, 16)]


@pytest.mark.parametrize("path,m,k,n,rank", LORA_CASES)
def test_lora_paths_match_oracle(gpu_lib, path, m, k, n, rank):
    import torch

    say("lora", path, m, k, n, rank, gpu_lib.describe_int4(m, n, k, path))
    d = int4_inputs(m, k, n, seed=600 + m + k + n)
    l = lora_inputs(k, n, rank, seed=700 + rank)
    t = upload_int4(d)
    la, lb = upload_lora(l)
    ref = oracle.qgemm_int4_lora(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"], l["lora_b"],
                                 2.0, m, k, n)
    y = gpu_lib.qgemm_int4_lora(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0, path=path)
    torch.cuda.synchronize()
    assert_accepted(host_u16(y), ref, ("lora", path, m, k, n, rank))
    # the smallest workspace (U and its slices only): no k split, no preparation pass
    lib = gpu_lib.load()
    up = lambda v: (v + 255) // 256 * 256
    u_bytes = (lib.qgemm_int4_lora_workspace_size(m, n, k, gpu_lib.PATHS[path])
               - up(gpu_lib.workspace_size(m, n, k, path)))
    u_only = torch.zeros(u_bytes, dtype=torch.uint8, device="cuda")
    y2 = gpu_lib.qgemm_int4_lora(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0, path=path,
                                 workspace=u_only)
    torch.cuda.synchronize()
    assert_accepted(host_u16(y2), ref, ("lora-min-ws", path, m, k, n, rank))


# (1024 x 1024 x 8192: the 256 x 128 tiles with U in the launch, 2^34 flops; 512 x 2048 x
# 8192: 128 x 128 tiles, U in the launch; 512 x 5120 x 25600: U in two small launches first;
# 16 x 8192 x 8192: the LDS-staged kernel over the whole k, U in the launch)
@pytest.mark.parametrize("m,k,n", [(1, 4096, 4096), (15, 2048, 8192), (512, 5120, 25600), (512, 2048, 8192),
                                   (1024, 1024, 8192), (8, 4096, 4096), (16, 8192, 8192)])
def test_lora_full_size_sampled(gpu_lib, m, k, n):
    import torch

    say("lora-full", m, k, n)
    d = int4_inputs(m, k, n, seed=900 + m)
    l = lora_inputs(k, n, 16, seed=901)
    t = upload_int4(d)
    la, lb = upload_lora(l)
    y = host_u16(gpu_lib.qgemm_int4_lora(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0))
    torch.cuda.synchronize()
    rows = sample_indices(m, 24, m)
    cols = sample_indices(n, 160, m + 1)
    ref = oracle.qgemm_int4_lora_at(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"], l["lora_b"],
                                    2.0, k, n, rows, cols)
    assert_accepted(y[np.ix_(rows, cols)], ref, ("lora-full", m, k, n))


# ----------------------------------------------------------------------------
# maximum sizes of the ABI: k = 2^22 (the 32-bit stage offsets' limit) on every
# path, and n = 2^26 columns (4 GiB of codes) on the GEMV and fused paths,
# checked on sampled columns
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("path,m", [("gemv", 1), ("fused", 8), ("mfma", 17), ("mfma_nows", 17)])
def test_max_k(gpu_lib, path, m):
    k, n = 1 << 22, 64
    p, ws = ("mfma", False) if path == "mfma_nows" else (path, None)
    say("max-k", path, m, k, n, gpu_lib.describe_int4(m, n, k, p, None if ws is None else 0))
    d = int4_inputs(m, k, n, seed=1100 + m)
    y = host_u16(run(gpu_lib, upload_int4(d), p, workspace=ws))
    cols = np.array([0, 1, 9, 31, 40, 63])
    ref = oracle.qgemm_int4_at(d["x"], d["qweight"], d["scales"], d["qzeros"], k, n, np.arange(m), cols)
    assert_accepted(y[:, cols], ref, ("max-k", path, m))


@pytest.mark.parametrize("path,m", [("gemv", 1), ("fused", 2)])
def test_max_n(gpu_lib, path, m):
    # 2^26 columns: operands drawn on the device from a seeded torch generator
    # (raw words and scale bit patterns of the same distributions), the sampled
    # columns copied back for the oracle
    import torch

    k, n = 128, 1 << 26
    say("max-n", path, m, k, n)
    g = torch.Generator(device="cuda")
    g.manual_seed(1200 + m)
    x = (torch.randn((m, k), generator=g, device="cuda")).to(torch.bfloat16)
    qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (k // 8, n), generator=g, device="cuda", dtype=torch.int32)
    sc = (0.005 + (torch.randn((1, n), generator=g, device="cuda") * 0.01).abs()).to(torch.float16)
    qz = torch.randint(-2 ** 31, 2 ** 31 - 1, (1, n // 8), generator=g, device="cuda", dtype=torch.int32)
    y = gpu_lib.qgemm_int4(x, qw, sc, qz, path=path)
    torch.cuda.synchronize()
    cols = np.array([0, 7, 8, 12345, (1 << 25) + 3, n - 9, n - 1])
    ct = torch.from_numpy(cols).cuda()
    xb = host_u16(x)
    qwb = host_u32(qw[:, ct])
    scb = host_u16(sc[:, ct])
    # zero words of the sampled columns, re-packed so that column j sits in nibble j % 8
    zw = host_u32(qz[:, ct // 8])
    zsel = ((zw >> (4 * (cols % 8)).astype(np.uint32)) & 0xF).astype(np.uint32) << (4 * (np.arange(len(cols)) % 8)).astype(np.uint32)
    # the oracle's zero layout packs 8 columns per word: rebuild words for the sample
    nq = (len(cols) + 7) // 8
    qzs = np.zeros((1, nq), dtype=np.uint32)
    for i in range(len(cols)):
        qzs[0, i // 8] |= np.uint32(zsel[0, i])
    pad = nq * 8 - len(cols)
    qwp = np.concatenate([qwb, np.zeros((k // 8, pad), dtype=np.uint32)], axis=1)
    scp = np.concatenate([scb, np.zeros((1, pad), dtype=np.uint16)], axis=1)
    ref = oracle.qgemm_int4(xb, qwp, scp, qzs, m, k, nq * 8)[:, :len(cols)]
    assert_accepted(host_u16(y[:, ct]), ref, ("max-n", path, m))


# ----------------------------------------------------------------------------
# fused epilogues (qgemm_int4_epilogue): the row reduction of an RMSNorm,
# row_sumsq[r] += sum_j y[r][j]^2 over the rounded outputs, with and without
# the LoRA add, on every kernel family (LDS-staged small-M, register-staged
# small-M with a k split and with row tiles, MFMA tiles with and without a k
# split); Y is bit-identical to the product without the reduction
# ----------------------------------------------------------------------------
EPI_CASES = [("gemv", 1, 1152, 776, 0), ("fused", 8, 2048, 1040, 0), ("fused", 15, 2048, 1040, 16),
             ("fused", 8, 16384, 520, 0), ("gemv", 1, 16384, 520, 16), ("auto", 24, 2048, 1040, 0),
             ("auto", 40, 2048, 1040, 5), ("mfma", 130, 1152, 776, 0), ("mfma", 33, 4096, 520, 16),
             ("mfma", 257, 2048, 1040, 0), ("fused", 3, 4096, 14336, 0), ("fused", 2, 20480, 4104, 16)]


@pytest.mark.parametrize("path,m,k,n,rank", EPI_CASES)
def test_epilogue_row_sumsq(gpu_lib, path, m, k, n, rank):
    import torch

    say("epilogue", path, m, k, n, rank, gpu_lib.describe_int4(m, n, k, path))
    d = int4_inputs(m, k, n, seed=1300 + m + k + n)
    t = upload_int4(d)
    rss = torch.zeros(m, dtype=torch.float32, device="cuda")
    if rank:
        l = lora_inputs(k, n, rank, seed=1400 + rank)
        la, lb = upload_lora(l)
        ref = oracle.qgemm_int4_lora(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"], l["lora_b"],
                                     2.0, m, k, n)
        y = gpu_lib.qgemm_int4_epilogue(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0,
                                        row_sumsq=rss, path=path)
        plain = gpu_lib.qgemm_int4_lora(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0, path=path)
    else:
        ref = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
        y = gpu_lib.qgemm_int4_epilogue(t["x"], t["qweight"], t["scales"], t["qzeros"], row_sumsq=rss,
                                        path=path)
        plain = gpu_lib.qgemm_int4(t["x"], t["qweight"], t["scales"], t["qzeros"], path=path)
    torch.cuda.synchronize()
    yb = host_u16(y)
    assert_accepted(yb, ref, ("epilogue", path, m, k, n, rank))
    assert np.array_equal(yb, host_u16(plain))
    got = rss.cpu().numpy().astype(np.float64)
    want, bound = oracle.row_sumsq(yb), oracle.row_sumsq_bound(yb)
    assert np.all(np.abs(got - want) <= bound), (np.max(np.abs(got - want) / np.maximum(bound, 1e-30)))
    # accumulated: a second call adds the same sums again
    if rank:
        gpu_lib.qgemm_int4_epilogue(t["x"], t["qweight"], t["scales"], t["qzeros"], la, lb, 2.0, row_sumsq=rss,
                                    out=y, path=path)
    else:
        gpu_lib.qgemm_int4_epilogue(t["x"], t["qweight"], t["scales"], t["qzeros"], row_sumsq=rss, out=y,
                                    path=path)
    torch.cuda.synchronize()
    got2 = rss.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got2 - 2 * want) <= 2 * bound + 2 * 2.0 ** -24 * 2 * want)


@pytest.mark.parametrize("m,k,n", [(15, 4096, 4096), (1, 4096, 28672), (512, 5120, 25600)])
def test_epilogue_row_sumsq_full_size(gpu_lib, m, k, n):
    import torch

    say("epilogue-full", m, k, n, gpu_lib.describe_int4(m, n, k))
    d = int4_inputs(m, k, n, seed=1500 + m)
    t = upload_int4(d)
    rss = torch.zeros(m, dtype=torch.float32, device="cuda")
    y = host_u16(gpu_lib.qgemm_int4_epilogue(t["x"], t["qweight"], t["scales"], t["qzeros"], row_sumsq=rss))
    torch.cuda.synchronize()
    rows, cols = sample_indices(m, 16, m), sample_indices(n, 96, m + 1)
    ref = oracle.qgemm_int4_at(d["x"], d["qweight"], d["scales"], d["qzeros"], k, n, rows, cols)
    assert_accepted(y[np.ix_(rows, cols)], ref, ("epilogue-full", m, k, n))
    got = rss.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - oracle.row_sumsq(y)) <= oracle.row_sumsq_bound(y))
