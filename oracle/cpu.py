"""ctypes binding of the C++ CPU oracle (qgemm_oracle_cpu.cpp) -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
use it.  The shared object is built in-tree with g++ (no HIP); ``build()``
compiles it and ``lib()`` compiles it once if nothing is built yet.  The
arguments are the raw storage arrays of the inputs (bf16/fp16 as uint16 bit
patterns, packed int4 as uint32 words); results are fp64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qgemm_oracle_cpu.cpp")
LIB = os.path.join(HERE, "liboracle_cpu.so")
CXX = os.environ.get("CXX_ORACLE", "g++")
LAYOUTS = {"NT": 0, "NN": 1, "TN": 2}
KINDS = {"fp16": 0, "bf16": 1}

_lib = None


def build() -> str:
    tmp = LIB + ".tmp"
    subprocess.run([CXX, "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-pthread", "-shared",
                    "-fPIC", SRC, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oc_hardware_threads.restype = ctypes.c_int
        L.oc_decode16.argtypes = [p, i64, i32, p]
        L.oc_dequant.argtypes = [p, p, p, i64, i64, i64, p]
        L.oc_dequant.restype = i32
        L.oc_qgemm_int4_at.argtypes = [p, i64, p, p, p, i64, i64, i64, i64, p, i64, p, i64, p, i32]
        L.oc_qgemm_int4_at.restype = i32
        L.oc_dense.argtypes = [i32, i32, i64, i64, i64, p, p, p, i32]
        L.oc_dense.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def hardware_threads() -> int:
    return int(lib().oc_hardware_threads())


def default_threads() -> int:
    """The host's CPU share: OMP_NUM_THREADS when set, else the hardware threads, at most 16."""
    env = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return env if env > 0 else min(16, hardware_threads())


def decode16(bits, kind: str) -> np.ndarray:
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib().oc_decode16(_ptr(b), b.size, KINDS[kind], _ptr(out))
    return out


def _check(rc, what):
    if rc == 1:
        raise AssertionError("%s: (q - z) * s is not exact in fp32" % what)
    if rc != 0:
        raise ValueError("%s: bad shape (status %d)" % (what, rc))


def dequant(qweight, scales, qzeros, k: int, n: int, group_size: int = 128) -> np.ndarray:
    """W32 [k][n] (fp32)."""
    qw, sc, qz = _c(qweight, np.uint32), _c(scales, np.uint16), _c(qzeros, np.uint32)
    w = np.empty((k, n), dtype=np.float32)
    _check(lib().oc_dequant(_ptr(qw), _ptr(sc), _ptr(qz), k, n, group_size, _ptr(w)), "dequant")
    return w


def qgemm_int4(x_bits, qweight, scales, qzeros, m: int, k: int, n: int, group_size: int = 128,
               rows=None, cols=None, threads: int = 0) -> np.ndarray:
    """Y64 [m][n] (or [len(rows)][len(cols)]) = X . W32 in fp64."""
    x = _c(x_bits, np.uint16)
    if x.ndim == 1:
        x = x.reshape(1, -1)
    ldx = x.shape[1] if x.size else k
    qw, sc, qz = _c(qweight, np.uint32), _c(scales, np.uint16), _c(qzeros, np.uint32)
    r = _c(rows, np.int64)
    c = _c(cols, np.int64)
    nr = m if r is None else r.size
    nc = n if c is None else c.size
    y = np.zeros((nr, nc), dtype=np.float64)
    if nr == 0 or nc == 0:
        return y
    _check(lib().oc_qgemm_int4_at(_ptr(x), ldx, _ptr(qw), _ptr(sc), _ptr(qz), m, k, n, group_size,
                                  _ptr(r), nr, _ptr(c), nc, _ptr(y), threads or default_threads()),
           "qgemm_int4")
    return y


def dense(layout: str, dtype: str, a_bits, b_bits, M: int, N: int, K: int, threads: int = 0) -> np.ndarray:
    """C64 [M][N] = op(A) . op(B) over the stored bf16/fp16 values."""
    a, b = _c(a_bits, np.uint16), _c(b_bits, np.uint16)
    c = np.zeros((M, N), dtype=np.float64)
    if M and N:
        _check(lib().oc_dense(LAYOUTS[layout], KINDS[dtype], M, N, K, _ptr(a), _ptr(b), _ptr(c),
                              threads or default_threads()), "dense")
    return c
