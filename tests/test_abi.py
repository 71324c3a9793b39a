"""C ABI contract checks that need no GPU: the library loads, exports every entry
point include/qgemm.h declares, and rejects invalid arguments with the exact
status code before anything is launched (no compute call is made here)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import int4_weight_only_gptq_amd as qg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")

OK, NULL, SHAPE, ALIGN, DTYPE, LAYOUT, UNSUP = 0, 1, 2, 3, 4, 5, 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^(?:int32_t|int64_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def defines(prefix):
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(%s\w*)\s+(\d+)" % prefix, text)}


@pytest.fixture(scope="module")
def lib():
    return qg.load()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "qg_abi_version", "qg_status_str", "qg_last_hip_error", "qgemm_int4", "qgemm_int4_path",
        "qgemm_int4_workspace_size", "qgemm_int4_describe", "qgemm_int4_dequant", "gemm_dense",
        "gemm_dense_batched", "qgemm_int4_lora", "qgemm_int4_lora_workspace_size", "qg_probe_mfma_bf16",
        "qg_probe_copy", "qg_probe_read", "qgemm_int4_noalloc", "qgemm_int4_epilogue", "qg_set_split_order",
        "qg_split_order", "gemm_dense_ws", "gemm_dense_workspace_size"])


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", qg.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_header_codes_match_binding():
    assert defines("QG_PATH_") == {"QG_PATH_AUTO": 0, "QG_PATH_GEMV": 1, "QG_PATH_FUSED": 2,
                                   "QG_PATH_MFMA": 3}
    assert {k: v for k, v in defines("QG_").items() if k in ("QG_NT", "QG_NN", "QG_TN")} == {
        "QG_NT": qg.LAYOUTS["NT"], "QG_NN": qg.LAYOUTS["NN"], "QG_TN": qg.LAYOUTS["TN"]}


def test_version_and_status_strings(lib):
    assert lib.qg_abi_version() == defines("QG_ABI")["QG_ABI_VERSION"]
    for code in range(9):
        assert lib.qg_status_str(code) and lib.qg_status_str(code) != b"unknown status"
    assert lib.qg_status_str(99) == b"unknown status"


# Fake device addresses: validation rejects the call before any use of them.
A16 = 0x10000          # 16-byte aligned
MIS = 0x10002          # 2-byte aligned only


def int4(lib, x=A16, ldx=256, qw=A16, sc=A16, qz=A16, y=A16, ldy=64, m=1, n=64, k=256, gs=128,
         path=0, ws=None, wsb=0):
    return lib.qgemm_int4_path(x, ldx, qw, sc, qz, y, ldy, m, n, k, gs, path, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(m=-1), SHAPE), (dict(n=-8), SHAPE), (dict(k=-128), SHAPE),
    (dict(gs=64), UNSUP), (dict(k=200), SHAPE), (dict(n=60), SHAPE),
    (dict(x=0), NULL), (dict(qw=0), NULL), (dict(sc=0), NULL), (dict(y=0), NULL),
    # qzeros NULL is valid (no zero point): the call gets past the pointer checks
    (dict(qz=0, x=MIS), ALIGN),
    (dict(ldx=128), SHAPE), (dict(ldy=32), SHAPE),
    (dict(x=MIS), ALIGN), (dict(ldx=260), ALIGN), (dict(qw=A16 + 4), ALIGN),
    (dict(sc=A16 + 2), ALIGN), (dict(qz=A16 + 2), ALIGN), (dict(y=A16 + 2), ALIGN),
    (dict(ldy=66), ALIGN),
    (dict(path=1, m=2), UNSUP), (dict(path=2, m=17), UNSUP), (dict(path=9), UNSUP),
    (dict(ws=A16 + 8, wsb=1024), ALIGN), (dict(wsb=-1), SHAPE),
    # 32-bit stage offsets: ldx and k at most 2^22, n at most 2^26
    (dict(ldx=(1 << 22) + 8), SHAPE), (dict(k=(1 << 22) + 128, ldx=(1 << 22) + 128), SHAPE),
    (dict(n=(1 << 26) + 8, ldy=(1 << 26) + 8), SHAPE),
])
def test_int4_rejects_invalid_arguments(lib, kw, code):
    assert int4(lib, **kw) == code


def lora(lib, x=A16, ldx=256, qw=A16, sc=A16, qz=A16, la=A16, lda=256, lb=A16, ldb=16, rank=16, y=A16,
         ldy=64, m=1, n=64, k=256, gs=128, path=0, ws=A16, wsb=1 << 20):
    return lib.qgemm_int4_lora(x, ldx, qw, sc, qz, la, lda, lb, ldb, rank, 1.0, y, ldy, m, n, k, gs, path,
                               ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(rank=0), SHAPE), (dict(rank=17), SHAPE), (dict(la=0), NULL), (dict(lb=0), NULL),
    (dict(lda=128), SHAPE), (dict(ldb=8), SHAPE), (dict(la=A16 + 8), ALIGN), (dict(lda=260), ALIGN),
    (dict(lda=(1 << 22) + 8), SHAPE),
    (dict(lb=A16 + 1), ALIGN), (dict(ws=None, wsb=0), SHAPE), (dict(wsb=32), SHAPE),
    (dict(x=MIS), ALIGN), (dict(gs=64), UNSUP), (dict(y=0), NULL),
    (dict(m=0, x=0, qw=0, sc=0, qz=0, la=0, lb=0, y=0, ws=None, wsb=0), OK),
])
def test_int4_lora_rejects_invalid_arguments(lib, kw, code):
    assert lora(lib, **kw) == code


def test_epilogue_rejects_invalid_arguments(lib):
    f = lib.qgemm_int4_epilogue
    # (x, ldx, qw, sc, qz, la, lda, lb, ldb, rank, scale, rss, y, ldy, m, n, k, gs, path, ws, wsb, stream)
    base = [A16, 256, A16, A16, A16, None, 0, None, 0, 0, 1.0, A16, A16, 64, 1, 64, 256, 128, 0, None, 0, None]
    assert f(*base[:11], A16 + 2, *base[12:]) == ALIGN                # misaligned row_sumsq
    args = list(base)
    args[16] = 200
    assert f(*args) == SHAPE                                          # k % 128
    args = list(base)
    args[0] = 0
    assert f(*args) == NULL
    args = list(base)
    args[14], args[0], args[2], args[3], args[4], args[12] = 0, 0, 0, 0, 0, 0
    assert f(*args) == OK                                             # m == 0: no-op
    # with an adapter: the LoRA checks (rank 17 is rejected)
    args = list(base)
    args[5], args[6], args[7], args[8], args[9], args[19], args[20] = A16, 256, A16, 16, 17, A16, 1 << 20
    assert f(*args) == SHAPE


def test_int4_lora_workspace_size(lib):
    for m, n, k in ((1, 4096, 4096), (15, 8192, 2048), (512, 25600, 5120), (33, 1040, 2048)):
        base = lib.qgemm_int4_workspace_size(m, n, k, 0)
        up = lambda v: (v + 255) // 256 * 256
        # U, then one 16 x 16 fp32 partial per row block and k slice (at most k / 512 slices)
        got = lib.qgemm_int4_lora_workspace_size(m, n, k, 0)
        blocks = (m + 15) // 16
        assert up(base) + up(64 * m) + 1024 * blocks <= got <= up(base) + up(64 * m) + 1024 * blocks * (k // 512)
    assert lib.qgemm_int4_lora_workspace_size(1, 64, 100, 0) < 0


def test_noalloc_validates_before_touching_the_device(lib):
    # the same argument checks as qgemm_int4, and problems whose workspace exceeds
    # the static scratch are rejected -- all before any HIP call
    f = lib.qgemm_int4_noalloc
    assert f(A16, 256, A16, A16, A16, A16, 64, 1, 64, 200, 128, None) == SHAPE
    assert f(0, 256, A16, A16, A16, A16, 64, 1, 64, 256, 128, None) == NULL
    assert f(MIS, 256, A16, A16, A16, A16, 64, 1, 64, 256, 128, None) == ALIGN
    assert f(A16, 256, A16, A16, A16, A16, 64, 1, 64, 256, 64, None) == UNSUP
    need = lib.qgemm_int4_workspace_size(2048, 5120, 25600, 0)
    assert need > defines("QG_NOALLOC")["QG_NOALLOC_SCRATCH_BYTES"] == 32 << 20
    assert f(A16, 25600, A16, A16, A16, A16, 5120, 2048, 5120, 25600, 128, None) == 8   # QG_ERR_SCRATCH
    assert f(0, 0, 0, 0, 0, 0, 0, 0, 64, 256, 128, None) == OK                          # m == 0: no-op


def test_int4_empty_problems_are_noops(lib):
    # m == 0 or n == 0: nothing is launched, NULL pointers allowed
    assert int4(lib, m=0, x=0, qw=0, sc=0, qz=0, y=0) == OK
    assert int4(lib, n=0, x=0, qw=0, sc=0, qz=0, y=0) == OK


def test_probe_rejects_invalid_arguments(lib):
    buf = ctypes.c_void_p(0x100000)
    assert lib.qg_probe_mfma_bf16(4, 10, None, None) == 1                     # NULL clocks
    assert lib.qg_probe_mfma_bf16(0, 10, buf, None) == 2                      # no workgroups
    assert lib.qg_probe_mfma_bf16(65537, 10, buf, None) == 2                  # too many
    assert lib.qg_probe_mfma_bf16(4, 0, buf, None) == 2                       # no iterations
    assert lib.qg_probe_mfma_bf16(4, 10, ctypes.c_void_p(0x100004), None) == 3  # misaligned


def test_split_order_setting(lib):
    assert defines("QG_SPLIT_ORDER_") == {"QG_SPLIT_ORDER_HW": qg.SPLIT_ORDERS["hw"],
                                          "QG_SPLIT_ORDER_ACQ_REL": qg.SPLIT_ORDERS["acq_rel"]}
    assert lib.qg_split_order() == 0                                           # the default
    try:
        assert lib.qg_set_split_order(1) == OK and lib.qg_split_order() == 1
        assert lib.qg_set_split_order(2) == UNSUP and lib.qg_split_order() == 1   # unchanged
        assert lib.qg_set_split_order(-1) == UNSUP
        qg.set_split_order("hw")
        assert qg.split_order() == "hw"
        with pytest.raises(KeyError):
            qg.set_split_order("seq_cst")
    finally:
        lib.qg_set_split_order(0)
    assert lib.qg_split_order() == 0


def test_dense_workspace_size(lib):
    # few tiles over a long k: min(4, 256 / tiles) slices of >= 1024 k of the 128 x 128 or
    # 256 x 128 tile (at most 128 tiles; the tile whose tiles x slices is larger, on a tie
    # 256 x 128 for NN and 128 x 128 for NT and TN; NT never 256 x 128): the counters (64 KiB)
    # then one fp32 BM x 128 partial tile per tile and slice
    t256, t128 = 256 * 128 * 4, 128 * 128 * 4
    assert qg.dense_workspace_size("NN", "bf16", 1024, 2048, 5632) == 65536 + 64 * 4 * t256   # tie: 256
    assert qg.dense_workspace_size("TN", "bf16", 1024, 2048, 5632) == 65536 + 128 * 2 * t128  # tie: 128
    assert qg.dense_workspace_size("TN", "fp16", 2048, 2048, 5632) == 65536 + 128 * 2 * t256  # 256 tiles of 128
    assert qg.dense_workspace_size("NN", "bf16", 512, 2048, 5632) == 65536 + 64 * 4 * t128    # 256 items > 128
    assert qg.dense_workspace_size("NT", "bf16", 1024, 2048, 5632) == 65536 + 128 * 2 * t128
    assert qg.dense_workspace_size("TN", "bf16", 200, 264, 4096) == 65536 + 6 * 4 * t128
    assert qg.dense_workspace_size("NT", "bf16", 520, 1000, 3072) == 65536 + 40 * 3 * t128   # 48 k tiles: 3 slices
    assert qg.dense_workspace_size("NN", "bf16", 520, 4000, 2048) == 65536 + 96 * 2 * t256
    # enough tiles, a short k, fp32, an unaligned contiguous extent, or an empty product: none
    for (lay, dt, M, N, K) in [("NT", "bf16", 4096, 2048, 5632), ("NN", "bf16", 1024, 5632, 2048),
                               ("NT", "bf16", 2048, 2048, 5632), ("NN", "bf16", 2560, 2048, 5632),
                               ("NT", "bf16", 520, 4000, 2048),
                               ("NT", "bf16", 1024, 2048, 1024), ("NT", "fp32", 1024, 2048, 5632),
                               ("NT", "bf16", 1024, 2048, 5630), ("NT", "bf16", 0, 2048, 5632),
                               ("NT", "bf16", 100, 2048, 5632)]:
        assert qg.dense_workspace_size(lay, dt, M, N, K) == 0, (lay, dt, M, N, K)
    assert lib.gemm_dense_workspace_size(3, 0, 8, 8, 8) == -LAYOUT
    assert lib.gemm_dense_workspace_size(0, 7, 8, 8, 8) == -DTYPE
    assert lib.gemm_dense_workspace_size(0, 0, -1, 8, 8) == -SHAPE


def test_dense_workspace_is_validated(lib):
    buf = 0x100000
    f = lib.gemm_dense_ws
    assert f(0, 0, 8, 8, 8, buf, 8, buf, 8, buf, 8, buf, -1, None) == SHAPE       # negative size
    assert f(0, 0, 8, 8, 8, buf, 8, buf, 8, buf, 8, buf + 8, 4096, None) == ALIGN   # misaligned
    assert f(3, 0, 8, 8, 8, buf, 8, buf, 8, buf, 8, None, 0, None) == LAYOUT
    assert f(0, 0, 8, 8, 8, None, 8, buf, 8, buf, 8, None, 0, None) == NULL


def test_bandwidth_probes_reject_invalid_arguments(lib):
    buf = 0x100000
    assert lib.qg_probe_copy(buf, buf + 4096, 100, 0, None) == SHAPE           # bytes % 16
    assert lib.qg_probe_copy(buf, buf + 4096, -16, 0, None) == SHAPE
    assert lib.qg_probe_copy(buf, buf + 4096, 64, 65537, None) == SHAPE        # too many workgroups
    assert lib.qg_probe_copy(None, buf, 64, 0, None) == NULL
    assert lib.qg_probe_copy(buf + 8, buf + 4096, 64, 0, None) == ALIGN
    assert lib.qg_probe_copy(None, None, 0, 0, None) == OK                     # nothing to do
    assert lib.qg_probe_read(buf, 64, 0, 1, None, None) == NULL                # NULL sink
    assert lib.qg_probe_read(buf, 64, -1, 1, buf + 4096, None) == SHAPE
    assert lib.qg_probe_read(buf, 64, 0, 1, buf + 4098, None) == ALIGN


def test_dequant_rejects_invalid_arguments(lib):
    d = lib.qgemm_int4_dequant
    assert d(A16, A16, A16, A16, 64, 100, 128, None) == SHAPE
    assert d(A16, A16, A16, A16, 64, 128, 32, None) == UNSUP
    assert d(0, A16, A16, A16, 64, 128, 128, None) == NULL
    assert d(A16, A16, A16, A16 + 4, 64, 128, 128, None) == ALIGN
    assert d(A16, A16, 0, A16 + 4, 64, 128, 128, None) == ALIGN     # qzeros NULL accepted
    assert d(A16, A16, A16, 0, 64, 128, 128, None) == NULL
    assert d(0, 0, 0, 0, 0, 128, 128, None) == OK


@pytest.mark.parametrize("args,code", [
    ((3, 0, 4, 4, 4, A16, 4, A16, 4, A16, 4), LAYOUT),
    ((0, 3, 4, 4, 4, A16, 4, A16, 4, A16, 4), DTYPE),
    ((0, 0, -1, 4, 4, A16, 4, A16, 4, A16, 4), SHAPE),
    ((0, 0, 4, 4, 4, 0, 4, A16, 4, A16, 4), NULL),
    ((0, 0, 4, 4, 4, A16, 4, A16, 4, 0, 4), NULL),
    ((0, 0, 4, 4, 4, A16, 3, A16, 4, A16, 4), SHAPE),      # NT: lda >= K
    ((2, 0, 8, 4, 4, A16, 4, A16, 4, A16, 4), SHAPE),      # TN: lda >= M
    ((1, 0, 4, 8, 4, A16, 4, A16, 4, A16, 8), SHAPE),      # NN: ldb >= N
    ((0, 0, 4, 4, 4, A16, 4, A16, 4, A16, 3), SHAPE),      # ldc >= N
    ((0, 0, 4, 4, 4, A16 + 1, 4, A16, 4, A16, 4), ALIGN),
    ((0, 0, 0, 4, 4, 0, 4, 0, 4, 0, 4), OK),
])
def test_dense_rejects_invalid_arguments(lib, args, code):
    assert lib.gemm_dense(*args, None) == code


def batched(lib, layout=0, dtype=0, batch=2, M=4, N=4, K=4, A=A16, lda=4, sa=16, B=A16, ldb=4, sb=16,
            C=A16, ldc=4, sc=16):
    return lib.gemm_dense_batched(layout, dtype, batch, M, N, K, A, lda, sa, B, ldb, sb, C, ldc, sc, None)


@pytest.mark.parametrize("kw,code", [
    (dict(layout=3), LAYOUT), (dict(dtype=3), DTYPE), (dict(batch=-1), SHAPE), (dict(batch=65536), SHAPE),
    (dict(sa=-1), SHAPE), (dict(sb=-16), SHAPE), (dict(sc=-16), SHAPE),
    (dict(sc=15), SHAPE),                       # outputs of consecutive products overlap
    (dict(A=0), NULL), (dict(C=0), NULL), (dict(lda=3), SHAPE), (dict(B=A16 + 1), ALIGN),
    (dict(batch=0, A=0, B=0, C=0), OK),         # nothing to do
    (dict(sc=15, batch=1, A=MIS + 1), ALIGN),   # batch 1: no overlap check
])
def test_dense_batched_rejects_invalid_arguments(lib, kw, code):
    assert batched(lib, **kw) == code


def test_dense_fp32_alignment_and_dtype(lib):
    # fp32 (dtype 2) needs 4-byte aligned pointers; dtype 3 does not exist
    assert lib.gemm_dense(0, 2, 4, 4, 4, A16 + 2, 4, A16, 4, A16, 4, None) == ALIGN
    assert lib.gemm_dense(0, 2, 4, 4, 4, A16, 4, A16, 4, A16 + 2, 4, None) == ALIGN
    assert lib.gemm_dense(0, 3, 4, 4, 4, A16, 4, A16, 4, A16, 4, None) == DTYPE
    assert lib.gemm_dense(0, 2, 0, 4, 4, 0, 4, 0, 4, 0, 4, None) == OK


def test_describe_names_the_dispatch(lib):
    # 4096 columns: 256 strips of 16, the LDS-staged kernel with 2 groups per wave
    # (16 waves over 32 groups); its LDS holds the strip's codes (32 groups x 1 KiB),
    # the activations (32 groups x 256 bytes) and the wave partial plane behind them
    # (16 waves x 1 token x 16 columns x 4 bytes)
    assert qg.describe_int4(1, 4096, 4096) == (
        "skinny_lds_kernel<1,dot,1,2,xlds> grid=256 block=1024 lds=%d ksplit=1 groups=32"
        % (32 * 1024 + 32 * 256 + 16 * 64))
    # 15 tokens: 4 KiB of activations per group (4 copies of 4 tokens x 256 bytes): 160 KiB
    # with the codes, so the partial plane reuses the codes' space
    assert qg.describe_int4(15, 4096, 4096) == (
        "skinny_lds_kernel<15,mfma,1,2,xlds> grid=256 block=1024 lds=%d ksplit=1 groups=32" % (160 * 1024))
    # 8192 columns: 256 strips of 32, one group per wave (16 groups)
    assert qg.describe_int4(8, 8192, 2048).startswith("skinny_lds_kernel<8,mfma,2,1,xlds> grid=256 block=1024")
    # more strips than one pass holds with all their codes in LDS: the register-staged kernel,
    # 224 strips of 128 columns (one 8-wave workgroup per CU) instead of 448 of 64; the GEMV
    # keeps 64-column strips
    assert qg.describe_int4(8, 28672, 4096).startswith("skinny_int4_kernel<8,mfma,8> grid=224 block=512")
    assert qg.describe_int4(16, 28672, 4096).startswith("skinny_int4_kernel<16,mfma,8> grid=224 block=512")
    assert qg.describe_int4(1, 28672, 4096).startswith("skinny_int4_kernel<1,dot,4> grid=448")
    # 64 groups would be split over 128 strips of 64 columns; instead 256 strips of 32
    # columns each take the whole k in the LDS-staged kernel (4 groups per wave, 16
    # waves): 64 groups x 2 KiB of codes and 16 waves x 16 tokens x 32 columns x 4 bytes
    assert qg.describe_int4(16, 8192, 8192) == (
        "skinny_lds_kernel<16,mfma,2,4,xreg> grid=256 block=1024 lds=%d ksplit=1 groups=64"
        % (64 * 2048 + 16 * 16 * 32 * 4))
    assert qg.describe_int4(8, 8192, 7168).startswith("skinny_lds_kernel<8,mfma,2,4,xreg> grid=256 block=896 ")
    assert qg.describe_int4(1, 5632, 8192).startswith("skinny_lds_kernel<1,dot,1,4,xreg> grid=352 block=1024 ")
    # 16-column strips with m >= 2 keep the split
    assert qg.describe_int4(8, 5632, 8192).startswith("skinny_int4_kernel<8,mfma,4> grid=264 ")
    # a long k with few strips is split: 200 groups over 40 strips of 128 columns in 256 / 40 =
    # 6 slices of 34 groups, one 512-thread workgroup per CU; where 128-column strips would keep
    # fewer than 20 groups per slice (112 groups over 32 strips: 8 slices of 14), 64-column
    # strips as before (m >= 8: 8-wave workgroups, 28 groups per slice over 64 strips)
    assert qg.describe_int4(16, 5120, 25600).startswith("skinny_int4_kernel<16,mfma,8> grid=240 block=512")
    assert "ksplit=6 groups=34" in qg.describe_int4(16, 5120, 25600)
    assert qg.describe_int4(16, 4096, 14336).startswith("skinny_int4_kernel<16,mfma,4> grid=256 block=512")
    assert "ksplit=4 groups=28" in qg.describe_int4(16, 4096, 14336)
    # the GEMV keeps 64-column strips; without a workspace no split and no 128-column strips
    assert qg.describe_int4(1, 5120, 25600).startswith("skinny_int4_kernel<1,dot,4> ")
    assert qg.describe_int4(16, 5120, 25600, workspace_bytes=0).startswith("skinny_int4_kernel<16,mfma,4> grid=80 ")
    assert "ksplit=1 groups=200" in qg.describe_int4(16, 5120, 25600, workspace_bytes=0)
    # pipelined MFMA kernel: 64-token tiles for small m, 256 x 128 once there are enough of them
    # (lds = 4 stages x (activations + words + metadata) dwords x 4 bytes)
    # pipelined MFMA kernel: tile and k split by rounds on 256 CUs (64 x 128 fits three to a
    # CU); with the workspace the activations are prepared and the group sums ride in the
    # metadata slots, without it a ones-MFMA per fragment and no split
    assert qg.describe_int4(17, 5120, 25600, path="mfma") == (
        "int4_pipe_kernel<64,128,4,prep> grid=320 block=128 lds=%d ksplit=8 groups=25"
        % (4 * (2048 + 1024 + 256) * 4))
    assert qg.describe_int4(17, 5120, 25600, path="mfma", workspace_bytes=0) == (
        "int4_pipe_kernel<128,128,4,ones> grid=40 block=256 lds=%d ksplit=1 groups=200"
        % (4 * (4096 + 1024 + 256) * 4))
    assert qg.describe_int4(2048, 25600, 5120) == (
        "int4_pipe_kernel<256,128,4,prep> grid=1600 block=512 lds=%d ksplit=1 groups=40"
        % (4 * (8192 + 1024 + 512) * 4))
    assert qg.describe_int4(512, 5120, 25600).startswith("int4_pipe_kernel<256,128,4,prep> grid=240 block=512")
    assert qg.describe_int4(2048, 5120, 25600, workspace_bytes=0).startswith(
        "int4_pipe_kernel<64,128,4,ones> grid=1280 block=128 lds=%d ksplit=1" % (4 * (2048 + 1024 + 128) * 4))
    # few tiles and a short k: 32 tiles of 64 x 128, k split into 8 slices of 4 groups
    assert qg.describe_int4(1, 4096, 4096, "mfma") == (
        "int4_pipe_kernel<64,128,4,prep> grid=256 block=128 lds=%d ksplit=8 groups=4" % (4 * (2048 + 1024 + 256) * 4))
    assert qg.describe_int4(0, 64, 128) == "none"
    assert qg.describe_int4(3, 64, 0) == "zero16_kernel"
    with pytest.raises(qg.QGemmError):
        qg.describe_int4(2, 64, 128, "gemv")


def test_workspace_size(lib):
    # 64 KiB of counters, then 40 strips x 6 slices x 16 tokens x 128 columns x 4 bytes
    assert qg.workspace_size(16, 5120, 25600) == 65536 + 40 * 6 * 16 * 128 * 4
    assert qg.workspace_size(8, 4096, 4096) == 0           # no split needed
    # MFMA tiles: 64 KiB of counters, prepared activations, group sums, then the k split's
    # partial tiles (tiles x slices x BM x 128 fp32)
    up = lambda b: (b + 255) // 256 * 256
    assert qg.workspace_size(2048, 25600, 5120) == up(65536 + 2048 * 5120 * 2 + 40 * 2048 * 4)  # no split
    desc = qg.describe_int4(17, 4096, 4096, path="mfma")
    bm = int(desc.split("<")[1].split(",")[0])
    ks = int(desc.split("ksplit=")[1].split()[0])
    tiles = ((17 + bm - 1) // bm) * (4096 // 128)
    assert ks > 1
    assert qg.workspace_size(17, 4096, 4096, path="mfma") == (
        up(65536 + 17 * 4096 * 2 + 32 * 17 * 4) + tiles * ks * bm * 128 * 4)
    # auto path, 16 < m <= 32 and n < 20480: the small-M kernel with two MFMA row tiles,
    # at most 8 waves (512 threads)
    assert qg.describe_int4(17, 4096, 4096).startswith("skinny_int4_kernel<17,mfma,1>")
    # more strips than CUs (352 here): the LDS-staged kernel with two groups per wave, so
    # that two 8-wave workgroups share a CU; 256 strips: one group per wave, 16 waves;
    # without the LDS-staged kernel (k split forced by a long k) the register-staged one
    assert qg.describe_int4(8, 5632, 2048).startswith("skinny_lds_kernel<8,mfma,1,2,xlds> grid=352 block=512 ")
    assert qg.describe_int4(8, 4096, 2048).startswith("skinny_lds_kernel<8,mfma,1,1,xlds> grid=256 block=1024 ")
    # two workgroups per CU leave no room for 15 tokens' activations: they stay in registers
    assert qg.describe_int4(15, 5632, 2048).startswith("skinny_lds_kernel<15,mfma,1,2,xreg> grid=352 block=512 ")
    assert qg.describe_int4(8, 5632, 20480).startswith("skinny_int4_kernel<8,mfma,")
    assert "block=512" in qg.describe_int4(32, 4096, 4096)
    assert qg.workspace_size(24, 5120, 25600) > 0
    # 32 < m <= 64: three or four row tiles when the workgroups fit one pass over the
    # 256 CUs (strips 32 columns wide up to 48 tokens, 16 above), else the MFMA tiles
    assert qg.describe_int4(33, 4096, 4096).startswith("skinny_int4_kernel<33,mfma,1> grid=256 ")
    assert qg.describe_int4(48, 8192, 2048).startswith("skinny_int4_kernel<48,mfma,2> grid=256 ")
    assert qg.describe_int4(64, 4096, 4096).startswith("skinny_int4_kernel<64,mfma,1> grid=256 ")
    assert qg.describe_int4(48, 14336, 4096).startswith("int4_pipe_kernel")   # 448 workgroups
    # two passes (at most 512 workgroups) only at k > 8192 and m <= 48
    assert qg.describe_int4(48, 4096, 14336).startswith("skinny_int4_kernel<48,mfma,2> grid=512 ")
    assert qg.describe_int4(33, 8192, 8192).startswith("int4_pipe_kernel")    # k = 8192: 512 workgroups
    assert qg.describe_int4(56, 4096, 14336).startswith("int4_pipe_kernel")
    assert qg.describe_int4(64, 8192, 2048).startswith("int4_pipe_kernel")    # 512 workgroups
    assert qg.describe_int4(65, 1024, 1024).startswith("int4_pipe_kernel")
    assert qg.describe_int4(17, 25600, 5120).startswith("skinny_int4_kernel<17,mfma,4>")   # m <= 24
    assert qg.describe_int4(32, 25600, 5120).startswith("skinny_int4_kernel<32,mfma,4> grid=400 ")  # 2 passes
    assert qg.describe_int4(32, 28672, 8192).startswith("int4_pipe_kernel")   # n >= 20480, 896 workgroups
    assert qg.describe_int4(32, 20472, 5120).startswith("skinny_int4_kernel<32,mfma,")
    assert lib.qgemm_int4_workspace_size(8, 60, 4096, 0) == -SHAPE
    assert lib.qgemm_int4_workspace_size(8, 64, 4096, 1) == -UNSUP


def test_library_has_no_undefined_kernel_symbols(lib):
    # a kernel whose host-side stub was dropped at compile time links but fails to load
    out = subprocess.run(["nm", "-D", "--undefined-only", qg.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    bad = [ln for ln in out.splitlines() if "qg" in ln or "device_stub" in ln]
    assert not bad, bad


def _parse_plan(desc):
    kv = dict(p.split("=") for p in desc.split()[1:] if "=" in p)
    return desc.split()[0], {k: int(v) for k, v in kv.items()}


def test_planned_launches_fit_the_hardware():
    # every plan the int4 dispatch can choose, over seeded random shapes and all paths:
    # a grid of at least one workgroup, at most 1024 threads, LDS within the 160 KiB of
    # a CU, k slices within the kernels' limits, and the workspace the plan was made
    # for is the size the library asks for
    rng = np.random.default_rng(20261203)
    shapes = [(1, 8, 128), (16, 8, 128), (17, 8, 128), (32, 20472, 128), (17, 20480, 128), (33, 20480, 25600)]   # (m, n, k)
    for _ in range(300):
        m = int(rng.choice([1, 2, 5, 8, 15, 16, 17, 24, 31, 32, 33, 40, 48, 49, 56, 64, 65, 100, 257, 512,
                            2048, 4097]))
        n = 8 * int(rng.integers(1, 4096))
        k = 128 * int(rng.integers(1, 256))
        shapes.append((m, n, k))
    for (m, n, k) in shapes:
        for path in ("auto", "gemv", "fused", "mfma"):
            if (path == "gemv" and m != 1) or (path == "fused" and m > 16):
                continue
            for ws in (None, 0):
                desc = qg.describe_int4(m, n, k, path, workspace_bytes=ws)
                name, p = _parse_plan(desc)
                what = (m, n, k, path, ws, desc)
                assert p["grid"] >= 1 and 64 <= p["block"] <= 1024 and p["block"] % 64 == 0, what
                assert 0 < p["lds"] <= 160 * 1024, what
                assert 1 <= p["ksplit"] <= 16 and p["groups"] >= 1, what
                assert p["ksplit"] * p["groups"] >= k // 128 > (p["ksplit"] - 1) * p["groups"], what
                if ws == 0:
                    assert p["ksplit"] == 1, what           # no workspace: no k split
                if name.startswith("skinny"):
                    assert p["grid"] % 8 == 0, what          # whole XCD rounds
                    if int(name.split("<")[1].split(",")[0]) > 16:
                        assert p["block"] <= 512, what       # __launch_bounds__(512) above 16 tokens
                    assert p["block"] // 64 <= p["groups"], what   # every wave has a group
                    if m > 32:   # row tiles in one pass, or two at long k
                        assert m <= 64 and (p["grid"] <= 256 or (m <= 48 and k > 8192 and p["grid"] <= 512)), what
