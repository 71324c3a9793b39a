"""Counter-based seeded generator for synthetic GEMM inputs (storage bytes only).

Definitions
-----------
* PRNG: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser as published by Vigna).  The
  i-th output (i = 1, 2, ...) of a stream seeded with s is
  mix(s + i * 0x9E3779B97F4A7C15 mod 2^64).
* Uniforms: the top 53 bits of a draw times 2^-53, in [0, 1).
* Gaussians: Box-Muller in fp64, one pair per two draws:
  r = sqrt(-2 ln(1 - u1)), z0 = r cos(2 pi u2), z1 = r sin(2 pi u2).
* bf16 storage: the fp64 value is rounded to fp32 (round to nearest even), then
  the fp32 bit pattern is rounded to its top 16 bits (round to nearest even).
* fp16 storage: fp64 rounded to IEEE binary16, round to nearest even.
* Packed int4 codes: a 4-bit code that is uniform on 0..15 for every nibble
  is the same thing as a uniform 32-bit word, so qweight and qzeros words are
  the top 32 bits of one draw each.  Nothing here unpacks or interprets them.

Workload values (the int4 recipe of the GPTQ linear layer and the dense
training products) are in `int4_inputs` and `dense_inputs`.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_C1 = np.uint64(0xBF58476D1CE4E5B9)
_C2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


class SplitMix64:
    """A SplitMix64 stream; every call continues where the last one stopped."""

    def __init__(self, seed: int):
        self.counter = 0
        self.seed = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)

    def u64(self, count: int) -> np.ndarray:
        out = np.empty(count, dtype=np.uint64)
        with np.errstate(over="ignore"):
            for start in range(0, count, _CHUNK):
                stop = min(count, start + _CHUNK)
                idx = np.arange(self.counter + start + 1, self.counter + stop + 1,
                                dtype=np.uint64)
                z = self.seed + idx * _GOLDEN
                z = (z ^ (z >> np.uint64(30))) * _C1
                z = (z ^ (z >> np.uint64(27))) * _C2
                out[start:stop] = z ^ (z >> np.uint64(31))
        self.counter += count
        return out

    def u32(self, count: int) -> np.ndarray:
        return (self.u64(count) >> np.uint64(32)).astype(np.uint32)

    def uniform(self, count: int) -> np.ndarray:
        return (self.u64(count) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)

    def normal(self, count: int) -> np.ndarray:
        pairs = (count + 1) // 2
        u = self.uniform(2 * pairs).reshape(pairs, 2)
        r = np.sqrt(-2.0 * np.log1p(-u[:, 0]))
        theta = 2.0 * np.pi * u[:, 1]
        z = np.empty((pairs, 2), dtype=np.float64)
        z[:, 0] = r * np.cos(theta)
        z[:, 1] = r * np.sin(theta)
        return z.reshape(-1)[:count]


def f32_to_bf16_bits(v) -> np.ndarray:
    """Round fp32 values (given as any float array) to bf16 bit patterns, RNE."""
    b = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32)
    b = b.astype(np.uint64)
    rounded = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def f64_to_fp16_bits(v) -> np.ndarray:
    """Round fp64 values to IEEE binary16 bit patterns, RNE."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def int4_inputs(m: int, k: int, n: int, seed: int, group_size: int = 128) -> dict:
    """Raw inputs of one int4 GPTQ product Y[m][n] = X[m][k] . W^T.

    Draw order: X, qweight, scales, qzeros.
      x        bf16 bits [m][k], values bf16(N(0, 1))
      qweight  uint32 [k/8][n], uniform words (8 uniform nibbles each)
      scales   fp16 bits [k/g][n], values fp16(0.005 + |N(0, 0.01)|)
      qzeros   uint32 [k/g][n/8], uniform words
    """
    if k % 8 or n % 8 or (group_size and k % group_size):
        raise ValueError("k must be a multiple of 8 and of the group size, n of 8")
    rng = SplitMix64(seed)
    groups = k // group_size if group_size else 0
    x = f32_to_bf16_bits(rng.normal(m * k)).reshape(m, k)
    qweight = rng.u32((k // 8) * n).reshape(k // 8, n)
    scales = f64_to_fp16_bits(0.005 + np.abs(0.01 * rng.normal(groups * n))).reshape(groups, n)
    qzeros = rng.u32(groups * (n // 8)).reshape(groups, n // 8)
    return {"x": x, "qweight": qweight, "scales": scales, "qzeros": qzeros,
            "m": m, "k": k, "n": n, "group_size": group_size}


def f64_to_fp32_bits(v) -> np.ndarray:
    """Round fp64 values to IEEE binary32 bit patterns, RNE."""
    return np.ascontiguousarray(np.asarray(v, dtype=np.float64).astype(np.float32)).view(np.uint32)


def normal_bits(rng: SplitMix64, shape, std: float, dtype: str) -> np.ndarray:
    """A tensor of N(0, std^2) values rounded to the storage dtype, as bit patterns."""
    count = int(np.prod(shape)) if len(shape) else 1
    v = std * rng.normal(count)
    if dtype == "fp32":
        bits = f64_to_fp32_bits(v)
    else:
        bits = f32_to_bf16_bits(v) if dtype == "bf16" else f64_to_fp16_bits(v)
    return bits.reshape(shape)


def dense_shapes(layout: str, M: int, N: int, K: int):
    """Storage shapes (row-major) of A and B for C[M][N] = op(A) op(B).

    NT: A[M][K], B[N][K];  NN: A[M][K], B[K][N];  TN: A[K][M], B[K][N].
    """
    if layout == "NT":
        return (M, K), (N, K)
    if layout == "NN":
        return (M, K), (K, N)
    if layout == "TN":
        return (K, M), (K, N)
    raise ValueError(layout)


def dense_inputs(layout: str, dtype: str, M: int, N: int, K: int, seed: int,
                 std: float = 0.02) -> dict:
    """Raw inputs of one dense product; draw order A then B, values N(0, std^2)."""
    rng = SplitMix64(seed)
    sa, sb = dense_shapes(layout, M, N, K)
    a = normal_bits(rng, sa, std, dtype)
    b = normal_bits(rng, sb, std, dtype)
    return {"a": a, "b": b, "layout": layout, "dtype": dtype, "M": M, "N": N, "K": K}


def dense_batched_inputs(layout: str, dtype: str, batch: int, M: int, N: int, K: int, seed: int,
                         std: float = 0.02) -> dict:
    """Raw inputs of `batch` dense products: a [batch][...] then b [batch][...], N(0, std^2)."""
    rng = SplitMix64(seed)
    sa, sb = dense_shapes(layout, M, N, K)
    a = normal_bits(rng, (batch,) + tuple(sa), std, dtype)
    b = normal_bits(rng, (batch,) + tuple(sb), std, dtype)
    return {"a": a, "b": b, "layout": layout, "dtype": dtype, "batch": batch, "M": M, "N": N, "K": K}


def lora_inputs(k: int, n: int, rank: int, seed: int, std_a: float = 0.02, std_b: float = 0.05) -> dict:
    """A LoRA adapter for an int4 layer: lora_a bf16 bits [rank][k] ~ N(0, std_a^2),
    then lora_b bf16 bits [n][rank] ~ N(0, std_b^2)."""
    rng = SplitMix64(seed)
    a = normal_bits(rng, (rank, k), std_a, "bf16")
    b = normal_bits(rng, (n, rank), std_b, "bf16")
    return {"lora_a": a, "lora_b": b, "rank": rank}
