"""Plain, slow, fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only tests/, the package smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the GPU library.

What it computes
----------------
* int4 GPTQ linear layer (the GPTQModel NF12 pull request, "What changed" and
  "Accuracy"; the mi50grad README, "Model": GPTQ-Int4 with group size 128).
  The weight of output column j at input row i is w = (q - z) * s, where q is
  the 4-bit code of (i, j), and z (4-bit) and s (fp16) are shared by the 128
  consecutive rows of i's group.  Storage:
    qweight uint32 [k/8][n]:   word (r, j) holds the codes of rows 8r..8r+7 of
                               column j, row 8r+t in bits 4t..4t+3;
    qzeros  uint32 [k/128][n/8]: word (g, c) holds the zeros of columns
                               8c..8c+7, column 8c+t in bits 4t..4t+3;
    scales  fp16   [k/128][n].
  Y[m][n] = X[m][k] . W, W[k][n] the dequantised weights.  The oracle forms W
  in fp32 (exact: |q - z| <= 15 has 4 bits and s has 11) and accumulates the
  products of the bf16 activations with it in fp64.
* the variant without a zero point (the mi50grad README, "Project Structure":
  an AWQ GEMV variant that skips the zero-point subtraction): w = q * s, the
  same storage without qzeros (passed as None here).
* dense products C = op(A) op(B) with fp32-accumulating bf16/fp16 inputs (the
  BC-250 tuned-GEMM post, "Where the time went" and "Checking the results are
  right": forward, input-gradient and weight-gradient products, each checked
  against a float64 product on the CPU).  Row-major layouts:
    NT: C[M][N] = A[M][K] . B[N][K]^T   (forward)
    NN: C[M][N] = A[M][K] . B[K][N]     (input gradient)
    TN: C[M][N] = A[K][M]^T . B[K][N]   (weight gradient)
  and batches of them (the batched products of attention layers), one product per
  leading index; and the same products in FP32 (the post tunes and validates
  FP32 in all three layouts), accepted under a dot-product error bound
  (accept_fp32).
* acceptance of an output y against the fp64 value r (the NF12 pull request,
  "Accuracy": zero violations of |err| <= 2e-3 + 2e-3 |ref|).  Read together
  with its statement that the rms error it sees is the BF16 rounding floor, an
  output is accepted when it meets that bound OR is one of the two output-dtype
  numbers that bracket r (a faithful rounding).  A correctly rounded bf16 value
  of a reference with |r| above about 2 can miss the literal bound, whose
  relative part is below bf16's half-ulp, so the literal formula alone would
  reject exact results.

Every floating-point decoding here is written from the IEEE field definitions,
not taken from a library conversion.
"""
from __future__ import annotations

import numpy as np

GROUP_SIZE = 128
TOL_ABS = 2e-3
TOL_REL = 2e-3

# significand bits (with the implicit one) and the smallest normal exponent
_GRID = {"bf16": (8, -126), "fp16": (11, -14)}


# ----------------------------------------------------------------------------
# IEEE decoders (fields -> value), fp64
# ----------------------------------------------------------------------------
def _decode(bits, exp_bits: int, man_bits: int) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64)
    bias = (1 << (exp_bits - 1)) - 1
    sign = np.where((b >> (exp_bits + man_bits)) & 1, -1.0, 1.0)
    e = (b >> man_bits) & ((1 << exp_bits) - 1)
    f = (b & ((1 << man_bits) - 1)).astype(np.float64)
    frac = f / float(1 << man_bits)
    with np.errstate(over="ignore", invalid="ignore"):
        normal = sign * (1.0 + frac) * np.exp2((e - bias).astype(np.float64))
        subnormal = sign * frac * np.exp2(float(1 - bias))
        special = np.where(f == 0, sign * np.inf, np.nan)
    top = (1 << exp_bits) - 1
    return np.where(e == 0, subnormal, np.where(e == top, special, normal))


def fp16_value(bits) -> np.ndarray:
    """IEEE binary16 bit patterns -> fp64 values (1 sign, 5 exponent, 10 fraction bits)."""
    return _decode(bits, 5, 10)


def bf16_value(bits) -> np.ndarray:
    """bfloat16 bit patterns -> fp64 values (1 sign, 8 exponent, 7 fraction bits)."""
    return _decode(bits, 8, 7)


def fp32_value(bits) -> np.ndarray:
    """IEEE binary32 bit patterns -> fp64 values (1 sign, 8 exponent, 23 fraction bits)."""
    return _decode(bits, 8, 23)


def _value(bits, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return fp32_value(bits)
    return bf16_value(bits) if dtype == "bf16" else fp16_value(bits)


# ----------------------------------------------------------------------------
# int4 GPTQ weights
# ----------------------------------------------------------------------------
def unpack_qweight(qweight, k: int, n: int) -> np.ndarray:
    """q[i][j] = floor(qweight[i // 8][j] / 16^(i mod 8)) mod 16, as int64 [k][n]."""
    qw = np.asarray(qweight, dtype=np.uint32).astype(np.int64)
    assert qw.shape == (k // 8, n)
    q = np.empty((k, n), dtype=np.int64)
    for t in range(8):
        q[t::8, :] = (qw // (16 ** t)) % 16
    return q


def unpack_qzeros(qzeros, groups: int, n: int) -> np.ndarray:
    """z[g][j] = floor(qzeros[g][j // 8] / 16^(j mod 8)) mod 16, as int64 [groups][n]."""
    qz = np.asarray(qzeros, dtype=np.uint32).astype(np.int64)
    assert qz.shape == (groups, n // 8)
    z = np.empty((groups, n), dtype=np.int64)
    for t in range(8):
        z[:, t::8] = (qz // (16 ** t)) % 16
    return z


def dequant(qweight, scales, qzeros, k: int, n: int, group_size: int = GROUP_SIZE,
            cols=None) -> np.ndarray:
    """W32[i][j] = fp32((q[i][j] - z[g][j]) * s[g][j]), g = i // group_size.

    qzeros None: no zero point, W32[i][j] = fp32(q[i][j] * s[g][j]).
    Returns fp32 [k][n] (or [k][len(cols)] for a column subset).  The product of a
    4-bit integer and an fp16 scale is exact in fp32; this is asserted.
    """
    groups = k // group_size
    qweight = np.asarray(qweight)
    scales = np.asarray(scales).reshape(groups, n)
    if cols is None:
        q = unpack_qweight(qweight, k, n)
        z = (np.zeros((groups, n), dtype=np.int64) if qzeros is None
             else unpack_qzeros(np.asarray(qzeros), groups, n))
        s = fp16_value(scales)
    else:
        # the same definitions, evaluated only for the requested columns
        cols = np.asarray(cols)
        q = unpack_qweight(qweight[:, cols], k, len(cols))
        if qzeros is None:
            z = np.zeros((groups, len(cols)), dtype=np.int64)
        else:
            zw = np.asarray(qzeros)[:, cols // 8].astype(np.int64)
            z = (zw // (16 ** (cols % 8))[None, :]) % 16
        s = fp16_value(scales[:, cols])
    g = np.arange(k) // group_size
    w64 = (q - z[g, :]).astype(np.float64) * s[g, :]
    w32 = w64.astype(np.float32)
    if not np.array_equal(w32.astype(np.float64), w64):
        raise AssertionError("(q - z) * s is not exact in fp32")
    return w32


def qgemm_int4(x_bits, qweight, scales, qzeros, m: int, k: int, n: int,
               group_size: int = GROUP_SIZE) -> np.ndarray:
    """Y64[m][n] = sum_i x[r][i] * W32[i][j], fp64 accumulation of bf16 x and fp32 W."""
    if m == 0 or n == 0:
        return np.zeros((m, n))
    if k == 0:
        return np.zeros((m, n))
    x = bf16_value(np.asarray(x_bits)[:, :k])
    w = dequant(qweight, scales, qzeros, k, n, group_size).astype(np.float64)
    return x @ w


def qgemm_int4_at(x_bits, qweight, scales, qzeros, k: int, n: int, rows, cols,
                  group_size: int = GROUP_SIZE) -> np.ndarray:
    """Y64 restricted to the given rows and columns: [len(rows)][len(cols)]."""
    x = bf16_value(np.asarray(x_bits)[np.asarray(rows), :k])
    w = dequant(qweight, scales, qzeros, k, n, group_size, cols=cols).astype(np.float64)
    return x @ w


def qgemm_int4_lora(x_bits, qweight, scales, qzeros, a_bits, b_bits, lora_scale: float, m: int, k: int,
                    n: int, group_size: int = GROUP_SIZE) -> np.ndarray:
    """Y64 = X . W + lora_scale * (X . A^T) . B^T, fp64 throughout.

    The int4 linear layer with a LoRA adapter added in its epilogue (the BC-250
    post's LoRA training, "Where the time went": rank-16 adapters on every
    linear layer; the mi50grad README, "Key Optimizations": a linear layer's
    epilogue fused into the same launch).  a_bits bf16 [r][k] (lora_A),
    b_bits bf16 [n][r] (lora_B); U = X . A^T is kept unrounded.
    """
    y = qgemm_int4(x_bits, qweight, scales, qzeros, m, k, n, group_size)
    if m == 0 or n == 0:
        return y
    x = bf16_value(np.asarray(x_bits)[:, :k])
    u = x @ bf16_value(a_bits).T
    return y + float(lora_scale) * (u @ bf16_value(b_bits).T)


def qgemm_int4_lora_at(x_bits, qweight, scales, qzeros, a_bits, b_bits, lora_scale: float, k: int, n: int,
                       rows, cols, group_size: int = GROUP_SIZE) -> np.ndarray:
    """qgemm_int4_lora restricted to the given rows and columns."""
    y = qgemm_int4_at(x_bits, qweight, scales, qzeros, k, n, rows, cols, group_size)
    x = bf16_value(np.asarray(x_bits)[np.asarray(rows), :k])
    u = x @ bf16_value(a_bits).T
    return y + float(lora_scale) * (u @ bf16_value(np.asarray(b_bits)[np.asarray(cols)]).T)


def row_sumsq(y_bits, dtype: str = "bf16") -> np.ndarray:
    """Per-row sum of squares of stored outputs, fp64: r[i] = sum_j y[i][j]^2.

    The reduction an RMSNorm takes over a linear layer's output row (the
    mi50grad README, "Key Optimizations": the fused GEMV + RMSNorm kernel sums
    the squares over the whole row), here of the rounded outputs as stored.
    """
    y = _value(np.asarray(y_bits), dtype)
    return np.sum(y * y, axis=-1)


def row_sumsq_bound(y_bits, dtype: str = "bf16") -> np.ndarray:
    """Bound on |fp32 sum - exact sum| for any order of adding the n squares in
    fp32 (each square rounded once, then n - 1 roundings of partial sums of
    nonnegative terms): (n + 1) * 2^-24 * sum_j y^2, plus the underflow floor."""
    y = _value(np.asarray(y_bits), dtype)
    n = y.shape[-1]
    return (n + 1) * 2.0 ** -24 * np.sum(y * y, axis=-1) + n * 2.0 ** -149


# ----------------------------------------------------------------------------
# dense products
# ----------------------------------------------------------------------------
def _ops(layout: str, a, b, dtype: str):
    A = _value(a, dtype)
    B = _value(b, dtype)
    if layout == "NT":
        return A, B.T
    if layout == "NN":
        return A, B
    if layout == "TN":
        return A.T, B
    raise ValueError(layout)


def dense(layout: str, dtype: str, a_bits, b_bits, M: int, N: int, K: int) -> np.ndarray:
    """C64[M][N] = op(A) . op(B) over the stored bf16/fp16 values, fp64."""
    opA, opB = _ops(layout, a_bits, b_bits, dtype)
    assert opA.shape == (M, K) and opB.shape == (K, N)
    if K == 0:
        return np.zeros((M, N))
    return opA @ opB


def dense_at(layout: str, dtype: str, a_bits, b_bits, rows, cols) -> np.ndarray:
    """C64 restricted to the given rows and columns."""
    opA, opB = _ops(layout, a_bits, b_bits, dtype)
    return opA[np.asarray(rows), :] @ opB[:, np.asarray(cols)]


def dense_absdot(layout: str, dtype: str, a_bits, b_bits, rows=None, cols=None) -> np.ndarray:
    """|op(A)| . |op(B)| in fp64 (optionally restricted): the scale of the fp32 error bound."""
    opA, opB = _ops(layout, a_bits, b_bits, dtype)
    if rows is not None:
        opA, opB = opA[np.asarray(rows), :], opB[:, np.asarray(cols)]
    return np.abs(opA) @ np.abs(opB)


def dense_batched(layout: str, dtype: str, a_bits, b_bits, M: int, N: int, K: int) -> np.ndarray:
    """C64[b] = op(A[b]) . op(B[b]) for b over the leading (batch) axis, fp64 [batch][M][N].

    The batched attention products of the BC-250 tuned-GEMM post ("Tuning the
    kernels", "Checking the results are right"): independent products of one
    shape, each defined as `dense`.
    """
    a_bits, b_bits = np.asarray(a_bits), np.asarray(b_bits)
    assert a_bits.shape[0] == b_bits.shape[0]
    out = np.zeros((a_bits.shape[0], M, N))
    for i in range(a_bits.shape[0]):
        out[i] = dense(layout, dtype, a_bits[i], b_bits[i], M, N, K)
    return out


def dense_batched_at(layout: str, dtype: str, a_bits, b_bits, index, rows, cols) -> np.ndarray:
    """C64[index] restricted to the given rows and columns."""
    return dense_at(layout, dtype, np.asarray(a_bits)[index], np.asarray(b_bits)[index], rows, cols)


# ----------------------------------------------------------------------------
# the output grid and the acceptance rule
# ----------------------------------------------------------------------------
def _ulp(r: np.ndarray, dtype: str) -> np.ndarray:
    p, emin = _GRID[dtype]
    mant, E = np.frexp(np.abs(r))   # |r| = mant * 2^E, mant in [0.5, 1)
    e = np.maximum(E.astype(np.int64) - 1, emin)
    return np.exp2((e - (p - 1)).astype(np.float64))


def grid_bracket(r, dtype: str):
    """The two output-dtype numbers lo <= r <= hi adjacent on that dtype's grid."""
    r = np.asarray(r, dtype=np.float64)
    u = _ulp(r, dtype)
    return np.floor(r / u) * u, np.ceil(r / u) * u


def round_to_grid(r, dtype: str) -> np.ndarray:
    """r rounded to the nearest output-dtype number, ties to even significand."""
    r = np.asarray(r, dtype=np.float64)
    u = _ulp(r, dtype)
    return np.rint(r / u) * u


def accept(y, r, dtype: str) -> np.ndarray:
    """Per element: |y - r| <= 2e-3 + 2e-3 |r|, or y is a faithful rounding of r."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    lo, hi = grid_bracket(r, dtype)
    literal = np.abs(y - r) <= TOL_ABS + TOL_REL * np.abs(r)
    return literal | (y == lo) | (y == hi)


# fp32 outputs (fp32 products and accumulation).  The pages validate FP32
# products against a float64 CPU product without stating a tolerance; the bound
# used is the classical one for a dot product of length K evaluated in
# floating point with unit roundoff u = 2^-24, in any order of summation:
#   |y - r| <= gamma_K * sum_i |a_i b_i|,   gamma_K = K u / (1 - K u),
# plus K times the smallest subnormal for underflow in the products.
def accept_fp32(y, r, absdot, K: int) -> np.ndarray:
    u = 2.0 ** -24
    gamma = K * u / (1.0 - K * u)
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return np.abs(y - r) <= gamma * np.asarray(absdot, dtype=np.float64) + K * 2.0 ** -149


def compare_fp32(y_bits, r, absdot, K: int) -> dict:
    """Compare fp32 output bit patterns with the fp64 reference under accept_fp32."""
    y = fp32_value(y_bits)
    r = np.asarray(r, dtype=np.float64)
    ok = accept_fp32(y, r, absdot, K)
    nr = float(np.sqrt(np.sum(r * r)))
    rms_rel = float(np.sqrt(np.sum((y - r) ** 2)) / nr) if nr > 0 else float(np.sqrt(np.sum(y * y)))
    return {"n": int(r.size), "rejected": int(r.size - np.count_nonzero(ok)), "rms_rel": rms_rel,
            "nonfinite": int(np.count_nonzero(~np.isfinite(y)))}


def compare(y_bits, r, dtype: str) -> dict:
    """Compare output bit patterns with the fp64 reference; summary statistics."""
    y = _value(y_bits, dtype)
    r = np.asarray(r, dtype=np.float64)
    ok = accept(y, r, dtype)
    literal = np.abs(y - r) <= TOL_ABS + TOL_REL * np.abs(r)
    nr = float(np.sqrt(np.sum(r * r)))
    rms_rel = float(np.sqrt(np.sum((y - r) ** 2)) / nr) if nr > 0 else float(
        np.sqrt(np.sum(y * y)))
    ulps = np.abs(y - round_to_grid(r, dtype)) / _ulp(r, dtype)
    return {
        "n": int(r.size),
        "rejected": int(r.size - np.count_nonzero(ok)),
        "literal_violations": int(r.size - np.count_nonzero(literal)),
        "rms_rel": rms_rel,
        "max_ulp": float(np.max(ulps)) if r.size else 0.0,
        "nonfinite": int(np.count_nonzero(~np.isfinite(y))),
    }
