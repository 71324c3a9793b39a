"""Python binding of the gfx950 int4 GPTQ / dense GEMM library (C ABI in include/qgemm.h).

Argument marshalling only: torch tensors supply device pointers, shapes and
strides, and torch's current HIP stream is passed through.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  The
library must have been built (``python -m int4_weight_only_gptq_amd.build``);
loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["load", "lib_path", "QGemmError", "qgemm_int4", "qgemm_int4_noalloc", "qgemm_int4_lora",
           "qgemm_int4_epilogue", "qgemm_int4_dequant", "gemm_dense",
           "gemm_dense_batched", "describe_int4",
           "workspace_size", "probe_mfma_bf16", "probe_copy", "probe_read",
           "abi_version", "PATHS", "LAYOUTS"]

_LIB_NAME = "libqgemm_gfx950.so"
_lib = None

PATHS = {"auto": 0, "gemv": 1, "fused": 2, "mfma": 3}
SPLIT_ORDERS = {"hw": 0, "acq_rel": 1}
LAYOUTS = {"NT": 0, "NN": 1, "TN": 2}
_DTYPES = {"bf16": 0, "fp16": 1, "fp32": 2}


class QGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.qg_status_str(status).decode() if _lib is not None else "status %d" % status
        if status == 7 and _lib is not None:
            msg += " (hipError %d)" % _lib.qg_last_hip_error()
        super().__init__("%s: %s" % (where, msg))
        self.status = status


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), _LIB_NAME)


def load():
    """Load the built library (binds to the HIP runtime torch has loaded)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- the library must share torch's HIP runtime

    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run python -m int4_weight_only_gptq_amd.build" % path)
    lib = ctypes.CDLL(path)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.qg_abi_version.restype = i32
    lib.qg_abi_version.argtypes = []
    lib.qg_status_str.restype = ctypes.c_char_p
    lib.qg_status_str.argtypes = [i32]
    lib.qg_last_hip_error.restype = i32
    lib.qg_last_hip_error.argtypes = []
    lib.qg_set_split_order.restype = i32
    lib.qg_set_split_order.argtypes = [i32]
    lib.qg_split_order.restype = i32
    lib.qg_split_order.argtypes = []
    int4_args = [vp, i64, vp, vp, vp, vp, i64, i64, i64, i64, i32]
    lib.qgemm_int4.restype = i32
    lib.qgemm_int4.argtypes = int4_args + [vp, i64, vp]
    lib.qgemm_int4_noalloc.restype = i32
    lib.qgemm_int4_noalloc.argtypes = int4_args + [vp]
    lib.qgemm_int4_path.restype = i32
    lib.qgemm_int4_path.argtypes = int4_args + [i32, vp, i64, vp]
    lib.qgemm_int4_workspace_size.restype = i64
    lib.qgemm_int4_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.qgemm_int4_describe.restype = i32
    lib.qgemm_int4_describe.argtypes = [i64, i64, i64, i32, i64, ctypes.c_char_p, i64]
    lib.qgemm_int4_dequant.restype = i32
    lib.qgemm_int4_dequant.argtypes = [vp, vp, vp, vp, i64, i64, i32, vp]
    lib.qgemm_int4_lora.restype = i32
    lib.qgemm_int4_lora.argtypes = [vp, i64, vp, vp, vp, vp, i64, vp, i64, i32, ctypes.c_float, vp, i64,
                                    i64, i64, i64, i32, i32, vp, i64, vp]
    lib.qgemm_int4_epilogue.restype = i32
    lib.qgemm_int4_epilogue.argtypes = [vp, i64, vp, vp, vp, vp, i64, vp, i64, i32, ctypes.c_float, vp, vp,
                                        i64, i64, i64, i64, i32, i32, vp, i64, vp]
    lib.qgemm_int4_lora_workspace_size.restype = i64
    lib.qgemm_int4_lora_workspace_size.argtypes = [i64, i64, i64, i32]
    lib.gemm_dense.restype = i32
    lib.gemm_dense.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.gemm_dense_ws.restype = i32
    lib.gemm_dense_ws.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    lib.gemm_dense_workspace_size.restype = i64
    lib.gemm_dense_workspace_size.argtypes = [i32, i32, i64, i64, i64]
    lib.gemm_dense_batched.restype = i32
    lib.gemm_dense_batched.argtypes = [i32, i32, i64, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64,
                                       i64, vp]
    lib.qg_probe_mfma_bf16.restype = i32
    lib.qg_probe_mfma_bf16.argtypes = [i64, i32, vp, vp]
    lib.qg_probe_copy.restype = i32
    lib.qg_probe_copy.argtypes = [vp, vp, i64, i64, vp]
    lib.qg_probe_read.restype = i32
    lib.qg_probe_read.argtypes = [vp, i64, i64, ctypes.c_uint32, vp, vp]
    _lib = lib
    return lib


def abi_version() -> int:
    return load().qg_abi_version()


def _stream(t, stream):
    import torch

    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    return torch.cuda.current_stream(t.device).cuda_stream


def _torch_stream(device, stream):
    """The launch stream as a torch stream object (the caller's, torch's current
    one, or a wrapper of a raw hipStream_t handle)."""
    import torch

    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream, device=device)
    return stream


def _ld(t) -> int:
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def _check(status, where):
    if status != 0:
        raise QGemmError(status, where)


_workspaces = {}


def set_split_order(order: str) -> None:
    """Ordering of the k split's partial-sum exchange, process-wide: "hw" (the
    default: agent-scope atomic partials behind a store-completion wait, relaxed
    ticket) or "acq_rel" (an acquire-release ticket; slower)."""
    _check(load().qg_set_split_order(SPLIT_ORDERS[order]), "qg_set_split_order")


def split_order() -> str:
    code = load().qg_split_order()
    return {v: k for k, v in SPLIT_ORDERS.items()}[code]


def workspace_size(m: int, n: int, k: int, path: str = "auto") -> int:
    """Bytes of workspace that let the m <= 16 paths split k (0 if none is used)."""
    size = load().qgemm_int4_workspace_size(m, n, k, PATHS[path])
    if size < 0:
        raise QGemmError(-size, "qgemm_int4_workspace_size")
    return size


def _workspace(device, stream, nbytes):
    """A zero-filled scratch tensor per (device, launch stream), grown on demand.

    It is allocated and zero-filled on the launch stream itself, so the fill is
    ordered before the kernels that read its counters, and the caching allocator
    hands a replaced buffer to later allocations on that stream only, after the
    kernels already queued there."""
    import torch

    if nbytes <= 0:
        return None
    ts = _torch_stream(device, stream)
    key = (device.index, ts.cuda_stream)
    t = _workspaces.get(key)
    if t is None or t.numel() < nbytes:
        with torch.cuda.stream(ts):
            t = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = t
    return t


def qgemm_int4(x, qweight, scales, qzeros, out=None, group_size: int = 128, path: str = "auto",
               workspace=None, stream=None):
    """Y[m][n] (bf16) = X[m][k] (bf16) . dequant(W)^T, W given in GPTQ int4 storage.

    qweight int32/uint32 [k/8][n]; scales fp16 [k/128][n]; qzeros int32/uint32
    [k/128][n/8], or None for weights without a zero point (w = q * s).
    ``path`` forces a kernel ("gemv", "fused", "mfma") or "auto".
    ``workspace``: None = a cached zero-filled buffer of the size the library
    asks for; False = no workspace (no k split); or a caller-owned uint8 tensor.
    """
    import torch

    lib = load()
    m, k = x.shape
    n = qweight.shape[1]
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    sh = _stream(x, stream)
    if workspace is None:
        workspace = _workspace(x.device, stream, workspace_size(m, n, k, path))
    if workspace is None or workspace is False:
        wptr, wbytes = None, 0
    else:
        wptr, wbytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = lib.qgemm_int4_path(x.data_ptr(), _ld(x), qweight.data_ptr(), scales.data_ptr(),
                             _ptr(qzeros), out.data_ptr(), _ld(out), m, n, k, group_size,
                             PATHS[path], wptr, wbytes, sh)
    _check(st, "qgemm_int4")
    return out


def qgemm_int4_noalloc(x, qweight, scales, qzeros, out, group_size: int = 128, stream=None):
    """qgemm_int4 through the entry point that allocates nothing: its workspace
    is the library's static per-GPU scratch (calls on one GPU must not overlap).
    ``out`` (bf16 [m][n]) is required, so this wrapper allocates nothing either."""
    import torch

    lib = load()
    m, k = x.shape
    n = qweight.shape[1]
    if x.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("x and out must be bfloat16")
    st = lib.qgemm_int4_noalloc(x.data_ptr(), _ld(x), qweight.data_ptr(), scales.data_ptr(), _ptr(qzeros),
                                out.data_ptr(), _ld(out), m, n, k, group_size, _stream(x, stream))
    _check(st, "qgemm_int4_noalloc")
    return out


def qgemm_int4_lora(x, qweight, scales, qzeros, lora_a, lora_b, lora_scale: float, out=None,
                    group_size: int = 128, path: str = "auto", workspace=None, stream=None):
    """qgemm_int4 plus a LoRA add in the epilogue: Y = X W + lora_scale (X A^T) B^T.

    lora_a bf16 [rank][k], lora_b bf16 [n][rank] (rank <= 16, last dimension
    contiguous).  ``workspace``: None = a cached buffer of
    qgemm_int4_lora_workspace_size bytes, or a caller-owned uint8 tensor (it
    must hold at least the fp32 [m][16] intermediate at its end)."""
    import torch

    lib = load()
    m, k = x.shape
    n = qweight.shape[1]
    rank = lora_a.shape[0]
    if x.dtype != torch.bfloat16 or lora_a.dtype != torch.bfloat16 or lora_b.dtype != torch.bfloat16:
        raise TypeError("x, lora_a and lora_b must be bfloat16")
    if lora_b.shape[1] < rank:
        raise ValueError("lora_b must be [n][rank]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    sh = _stream(x, stream)
    if workspace is None:
        size = lib.qgemm_int4_lora_workspace_size(m, n, k, PATHS[path])
        if size < 0:
            raise QGemmError(-size, "qgemm_int4_lora_workspace_size")
        workspace = _workspace(x.device, stream, size)
    wptr = None if workspace is None else workspace.data_ptr()
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.qgemm_int4_lora(x.data_ptr(), _ld(x), qweight.data_ptr(), scales.data_ptr(), _ptr(qzeros),
                             lora_a.data_ptr(), _ld(lora_a), lora_b.data_ptr(), _ld(lora_b), rank,
                             float(lora_scale), out.data_ptr(), _ld(out), m, n, k, group_size, PATHS[path],
                             wptr, wbytes, sh)
    _check(st, "qgemm_int4_lora")
    return out


def qgemm_int4_epilogue(x, qweight, scales, qzeros, lora_a=None, lora_b=None, lora_scale: float = 1.0,
                        row_sumsq=None, out=None, group_size: int = 128, path: str = "auto", workspace=None,
                        stream=None):
    """qgemm_int4 with the fused epilogues: the LoRA add (lora_a, lora_b given) and/or
    the row reduction row_sumsq[r] += sum_j y[r][j]^2 (fp32 [m] tensor, accumulated)."""
    import torch

    lib = load()
    m, k = x.shape
    n = qweight.shape[1]
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if row_sumsq is not None and (row_sumsq.dtype != torch.float32 or row_sumsq.numel() < m):
        raise TypeError("row_sumsq must be a float32 tensor of m elements")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    sh = _stream(x, stream)
    rank = 0 if lora_a is None else lora_a.shape[0]
    if workspace is None:
        size = (lib.qgemm_int4_lora_workspace_size(m, n, k, PATHS[path]) if lora_a is not None
                else lib.qgemm_int4_workspace_size(m, n, k, PATHS[path]))
        if size < 0:
            raise QGemmError(-size, "qgemm_int4_epilogue workspace size")
        workspace = _workspace(x.device, stream, size)
    wptr = None if workspace is None or workspace is False else workspace.data_ptr()
    wbytes = 0 if wptr is None else workspace.numel() * workspace.element_size()
    st = lib.qgemm_int4_epilogue(x.data_ptr(), _ld(x), qweight.data_ptr(), scales.data_ptr(), _ptr(qzeros),
                                 _ptr(lora_a), _ld(lora_a) if lora_a is not None else 0, _ptr(lora_b),
                                 _ld(lora_b) if lora_b is not None else 0, rank, float(lora_scale),
                                 _ptr(row_sumsq), out.data_ptr(), _ld(out), m, n, k, group_size, PATHS[path],
                                 wptr, wbytes, sh)
    _check(st, "qgemm_int4_epilogue")
    return out


def _ptr(t):
    return None if t is None else t.data_ptr()


def describe_int4(m: int, n: int, k: int, path: str = "auto", workspace_bytes=None) -> str:
    """Kernel and launch shape qgemm_int4 uses for (m, n, k, path); launches nothing."""
    lib = load()
    if workspace_bytes is None:
        workspace_bytes = workspace_size(m, n, k, path)
    buf = ctypes.create_string_buffer(256)
    _check(lib.qgemm_int4_describe(m, n, k, PATHS[path], workspace_bytes, buf, 256),
           "qgemm_int4_describe")
    return buf.value.decode()


def qgemm_int4_dequant(qweight, scales, qzeros, out=None, group_size: int = 128, stream=None):
    """fp32 [k][n] dequantised weights (q - z) * s (q * s when qzeros is None)."""
    import torch

    lib = load()
    k, n = qweight.shape[0] * 8, qweight.shape[1]
    if out is None:
        out = torch.empty((k, n), dtype=torch.float32, device=qweight.device)
    st = lib.qgemm_int4_dequant(qweight.data_ptr(), scales.data_ptr(), _ptr(qzeros),
                                out.data_ptr(), n, k, group_size, _stream(qweight, stream))
    _check(st, "qgemm_int4_dequant")
    return out


def _dtype_of(a, b):
    import torch

    names = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}
    if a.dtype != b.dtype or a.dtype not in names:
        raise TypeError("A and B must share dtype bf16, fp16 or fp32")
    return names[a.dtype]


def dense_workspace_size(layout: str, dtype: str, M: int, N: int, K: int) -> int:
    """Bytes of workspace that let gemm_dense split K for this product (0: no split)."""
    size = load().gemm_dense_workspace_size(LAYOUTS[layout], _DTYPES[dtype], M, N, K)
    if size < 0:
        raise QGemmError(-size, "gemm_dense_workspace_size")
    return size


def gemm_dense(layout: str, a, b, out=None, stream=None, workspace=None):
    """C = op(A) . op(B) for layout "NT", "NN" or "TN" (row-major, see qgemm.h);
    bf16 / fp16 with fp32 accumulation, or fp32 throughout.

    ``workspace``: None = the cached zero-filled buffer of the launch stream when
    the library asks for one (a k split for few-tile, long-K products); False =
    none; or a caller-owned uint8 tensor."""
    import torch

    lib = load()
    dtype = _dtype_of(a, b)
    if layout == "NT":
        (M, K), N = a.shape, b.shape[0]
    elif layout == "NN":
        (M, K), N = a.shape, b.shape[1]
    elif layout == "TN":
        (K, M), N = a.shape, b.shape[1]
    else:
        raise ValueError(layout)
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    if workspace is None:
        workspace = _workspace(a.device, stream, dense_workspace_size(layout, dtype, M, N, K))
    if workspace is None or workspace is False:
        st = lib.gemm_dense(LAYOUTS[layout], _DTYPES[dtype], M, N, K, a.data_ptr(), _ld(a),
                            b.data_ptr(), _ld(b), out.data_ptr(), _ld(out), _stream(a, stream))
    else:
        st = lib.gemm_dense_ws(LAYOUTS[layout], _DTYPES[dtype], M, N, K, a.data_ptr(), _ld(a),
                               b.data_ptr(), _ld(b), out.data_ptr(), _ld(out), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(), _stream(a, stream))
    _check(st, "gemm_dense")
    return out


def gemm_dense_batched(layout: str, a, b, out=None, stream=None):
    """C[i] = op(A[i]) . op(B[i]) for 3-D tensors [batch][rows][cols] (row-major per
    matrix, last dimension contiguous; any batch strides, 0 to reuse one operand)."""
    import torch

    lib = load()
    dtype = _dtype_of(a, b)
    if a.dim() != 3 or b.dim() != 3 or a.shape[0] != b.shape[0]:
        raise ValueError("A and B must be [batch][rows][cols] with the same batch")
    batch = a.shape[0]
    if layout == "NT":
        (M, K), N = a.shape[1:], b.shape[1]
    elif layout == "NN":
        (M, K), N = a.shape[1:], b.shape[2]
    elif layout == "TN":
        (K, M), N = a.shape[1:], b.shape[2]
    else:
        raise ValueError(layout)
    if out is None:
        out = torch.empty((batch, M, N), dtype=a.dtype, device=a.device)
    for t in (a, b, out):
        if t.shape[-1] > 1 and t.stride(-1) != 1:
            raise ValueError("last dimension must be contiguous")
    st = lib.gemm_dense_batched(LAYOUTS[layout], _DTYPES[dtype], batch, M, N, K,
                                a.data_ptr(), a.stride(1), a.stride(0), b.data_ptr(), b.stride(1),
                                b.stride(0), out.data_ptr(), out.stride(1), out.stride(0),
                                _stream(a, stream))
    _check(st, "gemm_dense_batched")
    return out


def probe_mfma_bf16(blocks: int, iters: int, clocks=None, stream=None):
    """Launch the register-resident bf16 MFMA probe (4 waves per workgroup, 8
    independent 16x16x32 MFMAs per wave per iteration: blocks * 4 * iters * 8 *
    16384 flops).  Returns the int64 [blocks][4] device tensor of clock stamps
    {shader cycles, constant counter} at start and end per workgroup."""
    import torch

    lib = load()
    if clocks is None:
        clocks = torch.zeros((blocks, 4), dtype=torch.int64, device="cuda")
    st = lib.qg_probe_mfma_bf16(blocks, iters, clocks.data_ptr(), _stream(clocks, stream))
    _check(st, "qg_probe_mfma_bf16")
    return clocks


def probe_copy(src, dst, nbytes=None, blocks: int = 0, stream=None):
    """16-byte lane copy of the first nbytes (default: all) of src into dst
    (measurement probe; both device tensors, 16-byte aligned)."""
    lib = load()
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    if nbytes > min(src.numel() * src.element_size(), dst.numel() * dst.element_size()):
        raise ValueError("nbytes exceeds a buffer")
    _check(lib.qg_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, blocks, _stream(src, stream)),
           "qg_probe_copy")


def probe_read(src, sink, nbytes=None, blocks: int = 0, key: int = 0x9E3779B9, stream=None):
    """16-byte lane read-only stream over the first nbytes (default: all) of src
    (measurement probe); sink is a device int32 tensor written only when a
    thread's XOR fold equals key."""
    lib = load()
    if nbytes is None:
        nbytes = src.numel() * src.element_size()
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds the buffer")
    _check(lib.qg_probe_read(src.data_ptr(), nbytes, blocks, key, sink.data_ptr(), _stream(src, stream)),
           "qg_probe_read")
