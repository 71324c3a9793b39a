"""GPU parity of the dense bf16/fp16 NT/NN/TN products against the CPU oracle.

Bar: zero rejections by the oracle's rule (|err| <= 2e-3 + 2e-3 |ref| or a
faithful rounding in the output dtype), no non-finite values, and rms_rel at
the rounding floor of the dtype (2.5e-3 bf16, 5e-4 fp16).
"""
import numpy as np
import pytest

import oracle
from oracle import cpu as cpp_oracle
from qgemm_inputs import dense_cases, dense_inputs, f32_to_bf16_bits, f64_to_fp16_bits

from gpu_helpers import dev, host_u16, sample_indices, say

pytestmark = pytest.mark.gpu

RMS_GATE = {"bf16": 2.5e-3, "fp16": 5e-4}


def tdtype(dtype):
    import torch

    return torch.bfloat16 if dtype == "bf16" else torch.float16


def run(qg, layout, a, b, out=None):
    import torch

    c = qg.gemm_dense(layout, a, b, out=out)
    torch.cuda.synchronize()
    return c


def assert_accepted(c_bits, ref, dtype, what):
    rep = oracle.compare(c_bits, ref, dtype)
    say(what, rep)
    assert rep["nonfinite"] == 0, (what, rep)
    assert rep["rejected"] == 0, (what, rep)
    if ref.size >= 64 and np.sqrt(np.mean(ref * ref)) > 0:
        assert rep["rms_rel"] < RMS_GATE[dtype], (what, rep)


SHAPES = [(1, 1, 1), (3, 5, 7), (16, 16, 16), (128, 128, 64), (130, 264, 200), (256, 136, 520),
          (64, 16, 1024), (16, 1024, 64), (1000, 8, 16)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_shapes_match_oracle(gpu_lib, layout, dtype):
    for i, (M, N, K) in enumerate(SHAPES):
        say("dense", layout, dtype, M, N, K)
        d = dense_inputs(layout, dtype, M, N, K, seed=500 + i)
        a, b = dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))
        c = host_u16(run(gpu_lib, layout, a, b))
        ref = cpp_oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
        assert_accepted(c, ref, dtype, (layout, dtype, M, N, K))


# shapes for the pipelined kernel (K % 64 == 0): ragged M and N edges, all four tile
# sizes (2050 x 5624 takes 256 x 256 tiles: one round of 198 against two of 396;
# 1000 x 2000 takes 64 x 128 tiles: one round of 256), two row bands, and the
# 128 x 128 tile over a long k (2048 x 2048 x 5632, the 2048-token forward and
# input-gradient products: 256 tiles in one round)
PIPE_SHAPES = [(128, 128, 64), (200, 264, 128), (1000, 136, 192), (2000, 2600, 64), (2050, 5624, 192),
               (1000, 2000, 128), (3000, 5632, 128),   # the last in two row bands (2816 + 184 rows)
               (2048, 2048, 5632)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_pipeline_shapes_match_oracle(gpu_lib, layout, dtype):
    import torch

    for i, (M, N, K) in enumerate(PIPE_SHAPES):
        say("pipe", layout, dtype, M, N, K)
        d = dense_inputs(layout, dtype, M, N, K, seed=700 + i)
        # without a workspace: no k split, the tiles as listed above
        c = host_u16(gpu_lib.gemm_dense(layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype)),
                                        workspace=False))
        torch.cuda.synchronize()
        if M * N <= 300000:
            ref = oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
            assert_accepted(c, ref, dtype, (layout, dtype, M, N, K))
        else:
            rows, cols = sample_indices(M, 96, i), sample_indices(N, 96, i + 1)
            ref = oracle.dense_at(layout, dtype, d["a"], d["b"], rows, cols)
            assert_accepted(c[np.ix_(rows, cols)], ref, dtype, (layout, dtype, M, N, K))


# the k split of gemm_dense_ws: few tiles over a long k, split into slices of >= 16 k tiles
# with a caller-owned workspace whose counters are zero again after every call; the same
# result twice and under both exchange orders; and without a workspace (no split) the
# oracle accepts it too.  The first four shapes split the 128 x 128 tile (4 tiles x 4
# slices; 6 ragged tiles x 4; 40 ragged tiles x 3; 6 ragged tiles x 4 slices of 17, 17, 17
# and 14 k tiles); the last has 160 such tiles, too many, so NN and TN split its 256 x 128
# tile (96 ragged tiles x 2, compared on sampled outputs) and NT does not split it at all
SPLIT_SHAPES = [(256, 256, 8192), (200, 264, 4096), (520, 1000, 3072), (200, 264, 4160), (520, 4000, 2048)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_k_split_matches_oracle(gpu_lib, layout, dtype):
    import torch

    for i, (M, N, K) in enumerate(SPLIT_SHAPES):
        need = gpu_lib.dense_workspace_size(layout, dtype, M, N, K)
        say("dense-split", layout, dtype, M, N, K, need)
        if i == 4 and layout == "NT":
            assert need == 0
            continue
        assert need > 65536
        d = dense_inputs(layout, dtype, M, N, K, seed=760 + i)
        a, b = dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))
        if M * N <= 600000:
            pick = lambda c: c
            ref = oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
        else:
            rows, cols = sample_indices(M, 96, i), sample_indices(N, 96, i + 1)
            pick = lambda c: c[np.ix_(rows, cols)]
            ref = oracle.dense_at(layout, dtype, d["a"], d["b"], rows, cols)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        c1 = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws))
        assert_accepted(pick(c1), ref, dtype, ("split", layout, dtype, M, N, K))
        assert int(torch.count_nonzero(ws[:65536])) == 0            # counters back at zero
        c2 = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws))
        assert np.array_equal(c1, c2)
        try:
            gpu_lib.set_split_order("acq_rel")
            c3 = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws))
        finally:
            gpu_lib.set_split_order("hw")
        assert np.array_equal(c1, c3)
        c0 = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=False))
        assert_accepted(pick(c0), ref, dtype, ("no-split", layout, dtype, M, N, K))
        # a workspace below the size asked for: no split either
        c4 = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws[:need - 256]))
        assert np.array_equal(c0, c4)


# the split with padded leading dimensions (16-byte multiples, so the pipelined tiles and
# the split still apply) and the output a view inside a larger buffer: the slices offset
# their k ranges through lda / ldb, and nothing outside the view is written
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_k_split_with_padded_leading_dims(gpu_lib, layout):
    import torch

    M, N, K = 200, 264, 4096
    say("dense-split-padded", layout, M, N, K)
    d = dense_inputs(layout, "bf16", M, N, K, seed=795)
    (ra, ca), (rb, cb) = d["a"].shape, d["b"].shape
    pa = torch.zeros((ra, ca + 24), dtype=torch.bfloat16, device="cuda")
    pb = torch.zeros((rb, cb + 40), dtype=torch.bfloat16, device="cuda")
    pa[:, 8:8 + ca] = dev(d["a"], torch.bfloat16)
    pb[:, 16:16 + cb] = dev(d["b"], torch.bfloat16)
    big = torch.full((M + 2, N + 24), 3.0, dtype=torch.bfloat16, device="cuda")
    out = big[1:M + 1, 8:8 + N]
    need = gpu_lib.dense_workspace_size(layout, "bf16", M, N, K)
    assert need > 65536
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    gpu_lib.gemm_dense(layout, pa[:, 8:8 + ca], pb[:, 16:16 + cb], out=out, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.dense(layout, "bf16", d["a"], d["b"], M, N, K)
    assert_accepted(host_u16(out), ref, "bf16", ("split-padded", layout))
    assert int(torch.count_nonzero(ws[:65536])) == 0
    g = big.float().cpu().numpy()
    g[1:M + 1, 8:8 + N] = 3.0
    assert np.all(g == 3.0)


# the split under HIP graph capture: one graph with a caller-owned workspace (zeroed before
# capture) and one with the binding's per-stream workspace (allocated and zero-filled inside
# the capture), each replayed three times with eager products on the same workspace in
# between; every replay gives the eager split result bit for bit and leaves the counters at zero
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_k_split_in_graph_replays(gpu_lib, layout):
    import torch

    M, N, K = 200, 264, 4096
    say("dense-split-graph", layout, M, N, K)
    d = dense_inputs(layout, "bf16", M, N, K, seed=790)
    a, b = dev(d["a"], torch.bfloat16), dev(d["b"], torch.bfloat16)
    need = gpu_lib.dense_workspace_size(layout, "bf16", M, N, K)
    assert need > 65536
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    want = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws))
    for own in (True, False):
        out = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gpu_lib.gemm_dense(layout, a, b, out=out, workspace=ws if own else None)
        for r in range(3):
            out.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(host_u16(out), want), ("replay", own, r)
            eager = host_u16(gpu_lib.gemm_dense(layout, a, b, workspace=ws))
            assert np.array_equal(eager, want)
        assert int(torch.count_nonzero(ws[:65536])) == 0
        del g


# shapes for the 16 x 16 split-k kernel (one of M, N <= 16, K >= 256): k tails
# inside a 32-row step, ragged 16-tiles, K not a multiple of 8 (TN only: K is
# then a row count), and both orientations of the skinny side
SPLITK_SHAPES = [(1000, 16, 2056), (16, 1000, 4104), (9, 24, 520), (40, 3, 1024), (24, 9, 1001),
                 (2048, 16, 256), (16, 16, 8200)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_splitk16_shapes_match_oracle(gpu_lib, layout, dtype):
    for i, (M, N, K) in enumerate(SPLITK_SHAPES):
        if K % 8 and layout != "TN":
            continue          # K is a contiguous dimension there; other kernels cover it
        say("splitk16", layout, dtype, M, N, K)
        d = dense_inputs(layout, dtype, M, N, K, seed=900 + i)
        c = host_u16(run(gpu_lib, layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))))
        ref = oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
        assert_accepted(c, ref, dtype, (layout, dtype, M, N, K))


# shapes for the K <= 32 outer-product kernel (NT and NN, M >= 64, N >= 256):
# ragged 64 x 256 tiles and waves past N, K below one 32-row step
SMALLK_SHAPES = [(64, 256, 16), (100, 264, 16), (130, 520, 24), (67, 1000, 8), (200, 304, 32)]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_smallk_shapes_match_oracle(gpu_lib, layout, dtype):
    for i, (M, N, K) in enumerate(SMALLK_SHAPES):
        say("smallk", layout, dtype, M, N, K)
        d = dense_inputs(layout, dtype, M, N, K, seed=950 + i)
        c = host_u16(run(gpu_lib, layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))))
        ref = oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
        assert_accepted(c, ref, dtype, (layout, dtype, M, N, K))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_pipeline_identity_is_exact(gpu_lib, layout):
    M = N = K = 256
    d = dense_inputs(layout, "bf16", M, N, K, seed=611, std=1.0)
    eye = f32_to_bf16_bits(np.eye(K))
    c = host_u16(run(gpu_lib, layout, dev(d["a"], tdtype("bf16")), dev(eye, tdtype("bf16"))))
    assert np.array_equal(c, d["a"] if layout != "TN" else d["a"].T)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_identity_is_exact(gpu_lib, layout):
    M = N = K = 136
    d = dense_inputs(layout, "bf16", M, N, K, seed=601, std=1.0)
    eye = f32_to_bf16_bits(np.eye(K))
    a = dev(d["a"], tdtype("bf16"))
    c = host_u16(run(gpu_lib, layout, a, dev(eye, tdtype("bf16"))))
    expect = d["a"] if layout != "TN" else d["a"].T
    assert np.array_equal(c, expect)


def test_fp16_subnormal_inputs(gpu_lib):
    # every A value subnormal; B = 2^k powers keep the products exact
    M, N, K = 32, 32, 64
    rng = np.random.default_rng(7)
    a = rng.integers(1, 0x400, size=(M, K)).astype(np.uint16)          # subnormal bit patterns
    b = f64_to_fp16_bits(2.0 ** rng.integers(0, 8, size=(N, K)))
    c = host_u16(run(gpu_lib, "NT", dev(a, tdtype("fp16")), dev(b, tdtype("fp16"))))
    ref = oracle.dense("NT", "fp16", a, b, M, N, K)
    assert_accepted(c, ref, "fp16", "subnormal")
    assert np.count_nonzero(c) > 0.9 * c.size


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_unaligned_and_strided_operands(gpu_lib, layout):
    import torch

    M, N, K = 37, 45, 53
    d = dense_inputs(layout, "bf16", M, N, K, seed=602)
    pa = torch.zeros((d["a"].shape[0], d["a"].shape[1] + 3), dtype=torch.bfloat16, device="cuda")
    pb = torch.zeros((d["b"].shape[0], d["b"].shape[1] + 5), dtype=torch.bfloat16, device="cuda")
    pa[:, 1:1 + d["a"].shape[1]] = dev(d["a"], torch.bfloat16)
    pb[:, 2:2 + d["b"].shape[1]] = dev(d["b"], torch.bfloat16)
    big = torch.full((M + 2, N + 6), 3.0, dtype=torch.bfloat16, device="cuda")
    out = big[1:M + 1, 3:3 + N]
    run(gpu_lib, layout, pa[:, 1:1 + d["a"].shape[1]], pb[:, 2:2 + d["b"].shape[1]], out=out)
    ref = oracle.dense(layout, "bf16", d["a"], d["b"], M, N, K)
    assert_accepted(host_u16(out), ref, "bf16", ("strided", layout))
    g = big.float().cpu().numpy()
    g[1:M + 1, 3:3 + N] = 3.0
    assert np.all(g == 3.0)


def test_k_zero_writes_zeros(gpu_lib):
    import torch

    a = torch.zeros((4, 0), dtype=torch.float16, device="cuda")
    b = torch.zeros((8, 0), dtype=torch.float16, device="cuda")
    out = torch.full((4, 8), 1.0, dtype=torch.float16, device="cuda")
    run(gpu_lib, "NT", a, b, out=out)
    assert torch.all(out == 0)


# ----------------------------------------------------------------------------
# the training trio at full size (t = 1024, 2048 and 4096), sampled outputs
# ----------------------------------------------------------------------------
FULL = [c for c in dense_cases(3) if c["t"] in (1024, 2048, 4096)]


@pytest.mark.parametrize("case", FULL, ids=["%s-%s-%s-t%d-w%dx%d" % (c["role"], c["layout"], c["dtype"], c["t"], *c["w"]) for c in FULL])
def test_training_products_sampled(gpu_lib, case):
    layout, dtype, M, N, K = case["layout"], case["dtype"], case["M"], case["N"], case["K"]
    say("trio", case)
    d = dense_inputs(layout, dtype, M, N, K, seed=case["seed"])
    c = host_u16(run(gpu_lib, layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))))
    rows = sample_indices(M, 48, case["seed"])
    cols = sample_indices(N, 48, case["seed"] + 1)
    ref = oracle.dense_at(layout, dtype, d["a"], d["b"], rows, cols)
    assert_accepted(c[np.ix_(rows, cols)], ref, dtype, case["role"])


# ----------------------------------------------------------------------------
# batched products (gemm_dense_batched): every kernel family, strided and
# broadcast operands, the attention workload at full size (sampled)
# ----------------------------------------------------------------------------
from qgemm_inputs import attention_cases, dense_batched_inputs  # noqa: E402

# (M, N, K) per kernel family: pipeline, 16-byte tile (K % 64 != 0), 16 x 16
# split-k, K <= 32 outer product, generic (unaligned)
BATCHED_SHAPES = [(200, 264, 128), (130, 136, 72), (1000, 16, 520), (100, 264, 16), (13, 17, 19)]


def run_batched(qg, layout, a, b, out=None):
    import torch

    c = qg.gemm_dense_batched(layout, a, b, out=out)
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_batched_shapes_match_oracle(gpu_lib, layout, dtype):
    for i, (M, N, K) in enumerate(BATCHED_SHAPES):
        if layout == "TN" and (M, N, K) == (100, 264, 16):
            continue      # the K <= 32 kernel is NT / NN; TN takes the tile path, covered above
        bt = 3
        say("batched", layout, dtype, bt, M, N, K)
        d = dense_batched_inputs(layout, dtype, bt, M, N, K, seed=1200 + i, std=0.5)
        c = host_u16(run_batched(gpu_lib, layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype))))
        ref = oracle.dense_batched(layout, dtype, d["a"], d["b"], M, N, K)
        for q in range(bt):
            assert_accepted(c[q], ref[q], dtype, ("batched", layout, dtype, q, M, N, K))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_batched_strided_broadcast_and_guarded_output(gpu_lib, layout):
    import torch

    bt, M, N, K = 4, 136, 144, 128
    d = dense_batched_inputs(layout, "bf16", bt, M, N, K, seed=1300, std=0.5)
    ra, ca = d["a"].shape[1:]
    rb, cb = d["b"].shape[1:]
    # A padded (rows and columns), B shared by every product (batch stride 0)
    pa = torch.zeros((bt, ra + 3, ca + 8), dtype=torch.bfloat16, device="cuda")
    pa[:, 1:ra + 1, :ca] = dev(d["a"], torch.bfloat16)
    a = pa[:, 1:ra + 1, :ca]
    b1 = dev(d["b"][:1], torch.bfloat16)
    b = b1.expand(bt, rb, cb)
    big = torch.full((bt, M + 2, N + 16), 7.0, dtype=torch.bfloat16, device="cuda")
    out = big[:, 1:M + 1, 8:8 + N]
    run_batched(gpu_lib, layout, a, b, out=out)
    bshared = np.repeat(d["b"][:1], bt, axis=0)
    ref = oracle.dense_batched(layout, "bf16", d["a"], bshared, M, N, K)
    got = host_u16(out)
    for q in range(bt):
        assert_accepted(got[q], ref[q], "bf16", ("strided", layout, q))
    g = big.float().cpu().numpy()
    g[:, 1:M + 1, 8:8 + N] = 7.0
    assert np.all(g == 7.0)


# all six products at 1024 tokens; the scores product (small operands, 1 GiB of
# output) at 4096
ATTN = [c for c in attention_cases()
        if c["dtype"] == "bf16" and (c["t"] == 1024 or (c["t"] == 4096 and c["role"] == "scores"))]


@pytest.mark.parametrize("case", ATTN, ids=["%s-%s-t%d" % (c["role"], c["layout"], c["t"]) for c in ATTN])
def test_attention_products_sampled(gpu_lib, case):
    layout, dtype, bt, M, N, K = case["layout"], case["dtype"], case["batch"], case["M"], case["N"], case["K"]
    say("attention", case)
    d = dense_batched_inputs(layout, dtype, bt, M, N, K, seed=case["seed"], std=1.0)
    out = run_batched(gpu_lib, layout, dev(d["a"], tdtype(dtype)), dev(d["b"], tdtype(dtype)))
    for q in (0, bt // 2, bt - 1):
        c = host_u16(out[q])
        rows = sample_indices(M, 24, case["seed"] + q)
        cols = sample_indices(N, 24, case["seed"] + q + 1)
        ref = oracle.dense_batched_at(layout, dtype, d["a"], d["b"], q, rows, cols)
        assert_accepted(c[np.ix_(rows, cols)], ref, dtype, (case["role"], q))


# ----------------------------------------------------------------------------
# FP32 products (fp32 in, fp32 products and accumulation, fp32 out): accepted
# under the dot-product error bound gamma_K * |A||B| (zero rejections), rms
# error at the fp32 floor
# ----------------------------------------------------------------------------
from gpu_helpers import host_u32  # noqa: E402

FP32_RMS_GATE = 2e-5
# the last shape takes the 128 x 128 tile (512 of them; 64-row tiles would need more rounds)
# with ragged rows, columns and k tile; the others take the 64-row tile or, unaligned, the
# one-thread-per-output kernel
FP32_SHAPES = [(1, 1, 1), (13, 17, 19), (128, 128, 64), (130, 264, 200), (256, 136, 520), (1000, 8, 16),
               (200, 264, 36), (64, 16, 1024), (2000, 4000, 100)]


def assert_fp32_accepted(c_bits, ref, absd, K, what):
    rep = oracle.compare_fp32(c_bits, ref, absd, K)
    say(what, rep)
    assert rep["nonfinite"] == 0, (what, rep)
    assert rep["rejected"] == 0, (what, rep)
    if ref.size >= 64:
        assert rep["rms_rel"] < FP32_RMS_GATE, (what, rep)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_fp32_shapes_match_oracle(gpu_lib, layout):
    import torch

    for i, (M, N, K) in enumerate(FP32_SHAPES):
        say("fp32", layout, M, N, K)
        d = dense_inputs(layout, "fp32", M, N, K, seed=1400 + i, std=1.0)
        c = host_u32(run(gpu_lib, layout, dev(d["a"], torch.float32), dev(d["b"], torch.float32)))
        ref = oracle.dense(layout, "fp32", d["a"], d["b"], M, N, K)
        absd = oracle.dense_absdot(layout, "fp32", d["a"], d["b"])
        assert_fp32_accepted(c, ref, absd, K, ("fp32", layout, M, N, K))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_fp32_batched_strided(gpu_lib, layout):
    import torch

    bt, M, N, K = 3, 136, 132, 72
    d = dense_batched_inputs(layout, "fp32", bt, M, N, K, seed=1500, std=1.0)
    ra, ca = d["a"].shape[1:]
    pa = torch.zeros((bt, ra + 1, ca + 4), dtype=torch.float32, device="cuda")
    pa[:, :ra, :ca] = dev(d["a"], torch.float32)
    big = torch.full((bt, M, N + 4), 5.0, dtype=torch.float32, device="cuda")
    out = big[:, :, 4:]
    run_batched(gpu_lib, layout, pa[:, :ra, :ca], dev(d["b"], torch.float32), out=out)
    got = host_u32(out)
    for q in range(bt):
        ref = oracle.dense(layout, "fp32", d["a"][q], d["b"][q], M, N, K)
        absd = oracle.dense_absdot(layout, "fp32", d["a"][q], d["b"][q])
        assert_fp32_accepted(got[q], ref, absd, K, ("fp32-batched", layout, q))
    assert torch.all(big[:, :, :4] == 5.0)


FP32_FULL = [c for c in dense_cases(3, with_lora=False) if c["dtype"] == "bf16" and c["t"] in (1024, 2048, 4096)]


@pytest.mark.parametrize("case", FP32_FULL,
                         ids=["%s-%s-t%d-w%dx%d" % (c["role"], c["layout"], c["t"], *c["w"]) for c in FP32_FULL])
def test_fp32_training_products_sampled(gpu_lib, case):
    import torch

    layout, M, N, K = case["layout"], case["M"], case["N"], case["K"]
    say("fp32-trio", case)
    d = dense_inputs(layout, "fp32", M, N, K, seed=case["seed"] + 7, std=0.02)
    c = host_u32(run(gpu_lib, layout, dev(d["a"], torch.float32), dev(d["b"], torch.float32)))
    rows = sample_indices(M, 48, case["seed"])
    cols = sample_indices(N, 48, case["seed"] + 1)
    ref = oracle.dense_at(layout, "fp32", d["a"], d["b"], rows, cols)
    absd = oracle.dense_absdot(layout, "fp32", d["a"], d["b"], rows, cols)
    assert_fp32_accepted(c[np.ix_(rows, cols)], ref, absd, K, ("fp32-trio", case["role"]))


# long reductions: the 16 x 16 split-k kernel over 2^19 k and the pipeline over
# 2^16 k (fp32 accumulation over long k stays inside the bound)
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("M,N,K", [(32, 16, 1 << 19), (256, 256, 1 << 16)])
def test_long_k(gpu_lib, layout, M, N, K):
    say("long-k", layout, M, N, K)
    d = dense_inputs(layout, "bf16", M, N, K, seed=1600 + M, std=0.02)
    c = host_u16(run(gpu_lib, layout, dev(d["a"], tdtype("bf16")), dev(d["b"], tdtype("bf16"))))
    rows, cols = sample_indices(M, 16, 1), sample_indices(N, 16, 2)
    ref = oracle.dense_at(layout, "bf16", d["a"], d["b"], rows, cols)
    assert_accepted(c[np.ix_(rows, cols)], ref, "bf16", ("long-k", layout, M, N, K))
