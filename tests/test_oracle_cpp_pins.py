"""Pins of the C++ CPU oracle (oracle/qgemm_oracle_cpu.cpp) against facts fixed by
the pages and by mathematics.

The same kinds of anchors as the numpy oracle's pins, none of them the oracle's
own formula: numpy's IEEE binary16 conversion and struct for the decoders,
hand-computed words and dequantised values (tests/golden/dequant_hand.txt),
brute force with exactly rounded sums (math.fsum), closed forms (one-hot rows,
blocked sums, identities, outer products) and the invariant q = z => Y = 0.
Agreement with the numpy oracle is checked last, on top of these pins.
"""
import math
import os
import struct

import numpy as np
import pytest

import oracle
from oracle import cpu
from qgemm_inputs import dense_inputs, f32_to_bf16_bits, f64_to_fp16_bits, int4_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(kind):
    with open(os.path.join(GOLDEN, "dequant_hand.txt")) as f:
        return [ln.split() for ln in f if ln.startswith(kind + " ")]


def _bf16_py(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _fp16_py(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


# ----------------------------------------------------------------------------
# decoders: all 65,536 patterns against numpy / the bf16 <-> fp32 bit relation
# ----------------------------------------------------------------------------
def test_fp16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = cpu.decode16(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(got[~np.isnan(got)]), np.signbit(ref[~np.isnan(ref)]))


def test_bf16_decoder_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint16)
    got = cpu.decode16(bits, "bf16")
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


# ----------------------------------------------------------------------------
# unpacking and dequantisation against hand values
# ----------------------------------------------------------------------------
def test_hand_words_through_dequant():
    # one word per column of an 8-row slice (k = 128 with the other rows zero),
    # s = 1, z = 0: W32 rows 0..7 are the codes of the word, low nibble first
    for parts in _golden_lines("word"):
        word = int(parts[1], 16)
        qw = np.zeros((16, 8), dtype=np.uint32)
        qw[0, :] = word
        qz = np.zeros((1, 1), dtype=np.uint32)
        sc = np.full((1, 8), 0x3C00, dtype=np.uint16)
        w = cpu.dequant(qw, sc, qz, 128, 8)
        assert w[:8, 0].tolist() == [float(v) for v in parts[2:]]
        assert np.all(w[8:] == 0)


def test_hand_zero_words_through_dequant():
    # codes all 15, s = 1: W32 of column c is 15 - z[c]
    for parts in _golden_lines("zeros"):
        word = int(parts[1], 16)
        qw = np.full((16, 8), 0xFFFFFFFF, dtype=np.uint32)
        qz = np.array([[word]], dtype=np.uint32)
        sc = np.full((1, 8), 0x3C00, dtype=np.uint16)
        w = cpu.dequant(qw, sc, qz, 128, 8)
        assert w[0].tolist() == [15.0 - int(v) for v in parts[2:]]


def test_dequant_hand_values():
    for parts in _golden_lines("w"):
        q, z, sbits, w = int(parts[1]), int(parts[2]), int(parts[3], 16), float(parts[5])
        qw = np.full((16, 8), q * 0x11111111, dtype=np.uint32)
        qz = np.full((1, 1), z * 0x11111111, dtype=np.uint32)
        sc = np.full((1, 8), sbits, dtype=np.uint16)
        got = cpu.dequant(qw, sc, qz, 128, 8)
        assert np.all(got == np.float32(w)), (parts, got[0, 0])


def test_dequant_without_zero_point_hand_values():
    for parts in _golden_lines("awq"):
        q, sbits, w = int(parts[1]), int(parts[2], 16), float(parts[4])
        qw = np.full((16, 8), q * 0x11111111, dtype=np.uint32)
        sc = np.full((1, 8), sbits, dtype=np.uint16)
        got = cpu.dequant(qw, sc, None, 128, 8)
        assert np.all(got == np.float32(w)), (parts, got[0, 0])


def test_orientation_and_group_index():
    # q[i][j] = i mod 8 (column 0) / 7 - i mod 8 (column 1); group 0: s = 0.5, z = 3;
    # group 1: s = 0.25, z = 15
    k, n = 256, 8
    qw = np.zeros((k // 8, n), dtype=np.uint32)
    qw[:, 0] = 0x76543210
    qw[:, 1] = 0x01234567
    qz = np.array([[0x33333333], [0xFFFFFFFF]], dtype=np.uint32)
    sc = np.array([[0x3800] * n, [0x3400] * n], dtype=np.uint16)
    w = cpu.dequant(qw, sc, qz, k, n)
    i = np.arange(k)
    q0, q1 = i % 8, 7 - i % 8
    s = np.where(i < 128, 0.5, 0.25)
    z = np.where(i < 128, 3, 15)
    assert np.array_equal(w[:, 0], ((q0 - z) * s).astype(np.float32))
    assert np.array_equal(w[:, 1], ((q1 - z) * s).astype(np.float32))


def test_shape_errors_are_reported():
    qw = np.zeros((16, 8), dtype=np.uint32)
    sc = np.zeros((1, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        cpu.dequant(qw, sc, None, 120, 8)       # k not a multiple of the group


# ----------------------------------------------------------------------------
# the int4 product: invariants, closed forms, brute force
# ----------------------------------------------------------------------------
def test_q_equals_z_gives_zero():
    k, n, m = 256, 32, 3
    d = int4_inputs(m, k, n, seed=51)
    qw = np.empty((k // 8, n), dtype=np.uint32)
    for j in range(n):
        for r in range(k // 8):
            z = (int(d["qzeros"][(8 * r) // 128, j // 8]) >> (4 * (j % 8))) & 15
            qw[r, j] = z * 0x11111111
    y = cpu.qgemm_int4(d["x"], qw, d["scales"], d["qzeros"], m, k, n)
    assert np.all(y == 0.0)


def test_one_hot_rows_select_weight_rows():
    k, n = 384, 24
    d = int4_inputs(1, k, n, seed=52)
    rows = [0, 7, 8, 127, 128, 200, 383]
    x = np.zeros((len(rows), k), dtype=np.uint16)
    for r, i in enumerate(rows):
        x[r, i] = 0x3F80
    y = cpu.qgemm_int4(x, d["qweight"], d["scales"], d["qzeros"], len(rows), k, n)
    for r, i in enumerate(rows):
        for j in range(n):
            q = (int(d["qweight"][i // 8, j]) >> (4 * (i % 8))) & 15
            z = (int(d["qzeros"][i // 128, j // 8]) >> (4 * (j % 8))) & 15
            assert y[r, j] == (q - z) * _fp16_py(d["scales"][i // 128, j])


def test_blocked_sum_closed_form():
    # X = 1 on group 1 only, q - z = 5 everywhere -> Y[j] = 128 * 5 * s[1][j]
    k, n = 384, 16
    d = int4_inputs(1, k, n, seed=53)
    x = np.zeros((1, k), dtype=np.uint16)
    x[0, 128:256] = 0x3F80
    qw = np.full((k // 8, n), 0x77777777, dtype=np.uint32)
    qz = np.full((k // 128, n // 8), 0x22222222, dtype=np.uint32)
    y = cpu.qgemm_int4(x, qw, d["scales"], qz, 1, k, n)
    s1 = d["scales"][1].view(np.float16).astype(np.float64)
    assert np.array_equal(y[0], 640.0 * s1)


@pytest.mark.parametrize("zeros", [True, False])
def test_brute_force_small_int4(zeros):
    m, k, n = 3, 256, 16
    d = int4_inputs(m, k, n, seed=54)
    qz = d["qzeros"] if zeros else None
    y = cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], qz, m, k, n)
    for r in range(m):
        for j in range(n):
            terms = []
            for i in range(k):
                q = (int(d["qweight"][i >> 3, j]) >> ((i & 7) << 2)) & 0xF
                z = (int(d["qzeros"][i >> 7, j >> 3]) >> ((j & 7) << 2)) & 0xF if zeros else 0
                terms.append(_bf16_py(d["x"][r, i]) * (q - z) * _fp16_py(d["scales"][i >> 7, j]))
            assert abs(y[r, j] - math.fsum(terms)) <= 1e-13 * max(1.0, abs(y[r, j])), (r, j)


def test_sampled_rows_and_columns_and_thread_count():
    m, k, n = 5, 512, 64
    d = int4_inputs(m, k, n, seed=55)
    full = cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n, threads=1)
    many = cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n, threads=7)
    assert np.array_equal(full, many)
    rows, cols = np.array([4, 0, 2]), np.array([63, 1, 8, 30])
    part = cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n, rows=rows, cols=cols)
    assert np.array_equal(part, full[np.ix_(rows, cols)])


def test_empty_shapes():
    d = int4_inputs(1, 128, 8, seed=56)
    assert cpu.qgemm_int4(d["x"][:0], d["qweight"], d["scales"], d["qzeros"], 0, 128, 8).shape == (0, 8)
    y = cpu.qgemm_int4(np.zeros((2, 0), np.uint16), d["qweight"][:0], d["scales"][:0], d["qzeros"][:0], 2, 0, 8)
    assert np.array_equal(y, np.zeros((2, 8)))


# ----------------------------------------------------------------------------
# dense products
# ----------------------------------------------------------------------------
def _store(v, dtype):
    v = np.asarray(v, dtype=np.float64)
    return f32_to_bf16_bits(v) if dtype == "bf16" else f64_to_fp16_bits(v)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_dense_brute_force(layout, dtype):
    M, N, K = 3, 4, 5
    d = dense_inputs(layout, dtype, M, N, K, seed=61, std=1.0)
    c = cpu.dense(layout, dtype, d["a"], d["b"], M, N, K)
    dec = _bf16_py if dtype == "bf16" else _fp16_py
    for i in range(M):
        for j in range(N):
            terms = []
            for p in range(K):
                a = d["a"][i, p] if layout in ("NT", "NN") else d["a"][p, i]
                b = d["b"][j, p] if layout == "NT" else d["b"][p, j]
                terms.append(dec(a) * dec(b))
            assert abs(c[i, j] - math.fsum(terms)) <= 1e-14 * max(1.0, abs(c[i, j]))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_dense_identity(layout):
    M = N = K = 16
    d = dense_inputs(layout, "fp16", M, N, K, seed=62, std=1.0)
    eye = _store(np.eye(K), "fp16")
    c = cpu.dense(layout, "fp16", d["a"], eye, M, N, K)
    a = d["a"].view(np.float16).astype(np.float64)
    assert np.array_equal(c, a if layout != "TN" else a.T)


def test_dense_k1_outer_product_and_1x1x1():
    a = _store([[2.0], [-3.0]], "fp16")
    b = _store([[0.5], [4.0], [1.0]], "fp16")
    assert cpu.dense("NT", "fp16", a, b, 2, 3, 1).tolist() == [[1.0, 8.0, 2.0], [-1.5, -12.0, -3.0]]
    one = _store([[1.5]], "bf16")
    assert cpu.dense("TN", "bf16", one, one, 1, 1, 1).tolist() == [[2.25]]


# ----------------------------------------------------------------------------
# the two oracles agree (each pinned on its own above and in test_oracle_pins.py)
# ----------------------------------------------------------------------------
def test_agrees_with_numpy_oracle():
    m, k, n = 4, 1152, 776
    d = int4_inputs(m, k, n, seed=57)
    w_cpp = cpu.dequant(d["qweight"], d["scales"], d["qzeros"], k, n)
    w_np = oracle.dequant(d["qweight"], d["scales"], d["qzeros"], k, n)
    assert np.array_equal(w_cpp.view(np.uint32), w_np.view(np.uint32))
    y_cpp = cpu.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    y_np = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    np.testing.assert_allclose(y_cpp, y_np, rtol=1e-12, atol=1e-12)
    for layout in ("NT", "NN", "TN"):
        dd = dense_inputs(layout, "bf16", 40, 24, 72, seed=58)
        np.testing.assert_allclose(cpu.dense(layout, "bf16", dd["a"], dd["b"], 40, 24, 72),
                                   oracle.dense(layout, "bf16", dd["a"], dd["b"], 40, 24, 72),
                                   rtol=1e-12, atol=1e-15)
