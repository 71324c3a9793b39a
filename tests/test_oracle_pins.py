"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every check here uses something other than the oracle's own formulas: IEEE
conversions of numpy / the struct module, hand-computed words, brute force with
exactly rounded sums (math.fsum), closed forms, invariants, and the error level
the GPTQModel NF12 pull request ("Accuracy") reports for a BF16-output path.
"""
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
from qgemm_inputs import (SplitMix64, f32_to_bf16_bits, f64_to_fp16_bits, int4_inputs, dense_inputs,
                          dense_batched_inputs, lora_inputs)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------
# generator
# ----------------------------------------------------------------------------
def test_splitmix64_published_sequence():
    # SplitMix64 with seed 0: the first outputs given with Vigna's reference code.
    assert [int(v) for v in SplitMix64(0).u64(3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_stream_continues():
    a = SplitMix64(77).u64(10)
    r = SplitMix64(77)
    b = np.concatenate([r.u64(3), r.u64(7)])
    assert np.array_equal(a, b)


def test_generator_distributions():
    d = int4_inputs(4, 1024, 512, seed=5)
    x = oracle.bf16_value(d["x"])
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1.0) < 0.05
    s = oracle.fp16_value(d["scales"])
    assert s.min() >= 0.005 and 0.01 < s.mean() < 0.02
    q = oracle.unpack_qweight(d["qweight"], 1024, 512)
    counts = np.bincount(q.reshape(-1), minlength=16)
    assert counts.min() > 0.9 * q.size / 16


# ----------------------------------------------------------------------------
# IEEE decoders against library conversions, exhaustively
# ----------------------------------------------------------------------------
def test_fp16_decoder_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.fp16_value(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_bf16_decoder_exhaustive():
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        ref = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = oracle.bf16_value(bits.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ----------------------------------------------------------------------------
# the output grid
# ----------------------------------------------------------------------------
def test_round_to_grid_matches_independent_rne():
    rng = SplitMix64(3)
    v = np.concatenate([rng.normal(20000) * 10.0 ** rng.normal(20000),
                        rng.normal(2000) * 1e-39, rng.normal(2000) * 1e-6])
    v32 = v.astype(np.float32).astype(np.float64)
    # bf16: the generator's bit-level RNE on fp32 bit patterns
    assert np.array_equal(oracle.round_to_grid(v32, "bf16"),
                          oracle.bf16_value(f32_to_bf16_bits(v32)))
    # fp16: numpy's IEEE conversion
    vv = v[np.abs(v) < 60000]
    assert np.array_equal(oracle.round_to_grid(vv, "fp16"), vv.astype(np.float16).astype(np.float64))


def test_grid_bracket_hand_values():
    lo, hi = oracle.grid_bracket(np.array([1.0, 1 + 2 ** -9, -(1 + 2 ** -9), 0.0]), "bf16")
    assert list(lo) == [1.0, 1.0, -(1 + 2 ** -7), 0.0]
    assert list(hi) == [1.0, 1 + 2 ** -7, -1.0, 0.0]
    lo, hi = oracle.grid_bracket(np.array([1 + 2 ** -12, 2 ** -25]), "fp16")
    assert list(lo) == [1.0, 0.0] and list(hi) == [1 + 2 ** -10, 2 ** -24]
    # ties go to the even significand
    assert oracle.round_to_grid(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8]), "bf16").tolist() == [
        1.0, 1 + 2 ** -6]


def test_accept_rule():
    r = np.array([3.0 + 2 ** -8, 3.0 + 2 ** -8, 100.0, 1e-4])
    y = np.array([3.0, 3.0 + 2 ** -6, 100.0 + 0.75, 1e-4 + 1.9e-3])
    # 3.0 and 3.0 + 2^-6 bracket 3 + 2^-8 on the bf16 grid; 100.75 is neither
    # within the bound nor a bracket (brackets of 100 are 100); the last is
    # within the absolute part of the bound.
    assert oracle.accept(y, r, "bf16").tolist() == [True, True, False, True]
    assert not oracle.accept(np.array([np.nan]), np.array([1.0]), "bf16")[0]


# ----------------------------------------------------------------------------
# int4 storage: unpacking and dequantisation against hand values
# ----------------------------------------------------------------------------
def _golden_lines(kind):
    with open(os.path.join(GOLDEN, "dequant_hand.txt")) as f:
        return [ln.split() for ln in f if ln.startswith(kind + " ")]


def test_unpack_qweight_hand_words():
    for parts in _golden_lines("word"):
        word = int(parts[1], 16)
        q = oracle.unpack_qweight(np.array([[word]], dtype=np.uint32), 8, 1)[:, 0]
        assert q.tolist() == [int(v) for v in parts[2:]]


def test_unpack_qweight_orientation():
    # two word-rows, two columns: rows 0..7 come from word-row 0, 8..15 from 1
    qw = np.array([[0x76543210, 0x01234567], [0xFEDCBA98, 0x89ABCDEF]], dtype=np.uint32)
    q = oracle.unpack_qweight(qw, 16, 2)
    assert q[:, 0].tolist() == list(range(16))
    assert q[:, 1].tolist() == [7, 6, 5, 4, 3, 2, 1, 0, 15, 14, 13, 12, 11, 10, 9, 8]


def test_unpack_qzeros_hand_words():
    for parts in _golden_lines("zeros"):
        word = int(parts[1], 16)
        z = oracle.unpack_qzeros(np.array([[word]], dtype=np.uint32), 1, 8)[0]
        assert z.tolist() == [int(v) for v in parts[2:]]


def test_dequant_hand_values():
    for parts in _golden_lines("w"):
        q, z, sbits, w = int(parts[1]), int(parts[2]), int(parts[3], 16), float(parts[5])
        qw = np.full((16, 8), q * 0x11111111, dtype=np.uint32)
        qz = np.full((1, 1), z * 0x11111111, dtype=np.uint32)
        sc = np.full((1, 8), sbits, dtype=np.uint16)
        got = oracle.dequant(qw, sc, qz, 128, 8)
        assert np.all(got == np.float32(w)), (parts, got[0, 0])


def test_dequant_without_zero_point_hand_values():
    for parts in _golden_lines("awq"):
        q, sbits, w = int(parts[1]), int(parts[2], 16), float(parts[4])
        qw = np.full((16, 8), q * 0x11111111, dtype=np.uint32)
        sc = np.full((1, 8), sbits, dtype=np.uint16)
        got = oracle.dequant(qw, sc, None, 128, 8)
        assert np.all(got == np.float32(w)), (parts, got[0, 0])
        sub = oracle.dequant(qw, sc, None, 128, 8, cols=np.array([3, 5]))
        assert np.all(sub == np.float32(w))


def test_dequant_group_index():
    # k = 256: group 0 (rows 0..127) has s = 0.5, z = 3; group 1 s = 0.25, z = 15
    k, n = 256, 8
    qw = np.full((k // 8, n), 0x76543210, dtype=np.uint32)   # q[i][j] = i mod 8
    qz = np.array([[0x33333333], [0xFFFFFFFF]], dtype=np.uint32)
    sc = np.array([[0x3800] * n, [0x3400] * n], dtype=np.uint16)
    w = oracle.dequant(qw, sc, qz, k, n)
    i = np.arange(k)
    expect = np.where(i < 128, (i % 8 - 3) * 0.5, (i % 8 - 15) * 0.25)
    assert np.array_equal(w, np.repeat(expect[:, None], n, axis=1).astype(np.float32))


def test_dequant_zero_column_index():
    # zeros differ per column: z = column index mod 8 (word 0x76543210)
    k, n = 128, 16
    qw = np.full((k // 8, n), 0xFFFFFFFF, dtype=np.uint32)   # q = 15
    qz = np.full((1, n // 8), 0x76543210, dtype=np.uint32)
    sc = np.full((1, n), 0x3C00, dtype=np.uint16)           # s = 1
    w = oracle.dequant(qw, sc, qz, k, n)
    assert np.array_equal(w[0], (15 - np.arange(n) % 8).astype(np.float32))


# ----------------------------------------------------------------------------
# the int4 product: invariants, closed forms and brute force
# ----------------------------------------------------------------------------
def _z_matching_qweight(qzeros, k, n):
    """qweight whose every code equals its column's zero (so w = 0)."""
    qw = np.empty((k // 8, n), dtype=np.uint32)
    for j in range(n):
        for r in range(k // 8):
            g = (8 * r) // 128
            z = (int(qzeros[g, j // 8]) >> (4 * (j % 8))) & 15
            qw[r, j] = z * 0x11111111
    return qw


def test_q_equals_z_gives_zero():
    d = int4_inputs(3, 256, 32, seed=11)
    qw = _z_matching_qweight(d["qzeros"], 256, 32)
    y = oracle.qgemm_int4(d["x"], qw, d["scales"], d["qzeros"], 3, 256, 32)
    assert np.all(y == 0.0)


def test_one_hot_rows_select_weight_rows():
    k, n = 384, 24
    d = int4_inputs(1, k, n, seed=12)
    rows = [0, 7, 8, 127, 128, 200, 383]
    x = np.zeros((len(rows), k), dtype=np.uint16)
    for r, i in enumerate(rows):
        x[r, i] = 0x3F80                      # bf16 1.0
    y = oracle.qgemm_int4(x, d["qweight"], d["scales"], d["qzeros"], len(rows), k, n)
    # independent per-element dequant from the storage definition
    for r, i in enumerate(rows):
        for j in range(n):
            q = (int(d["qweight"][i // 8, j]) >> (4 * (i % 8))) & 15
            z = (int(d["qzeros"][i // 128, j // 8]) >> (4 * (j % 8))) & 15
            s = struct.unpack("<e", struct.pack("<H", int(d["scales"][i // 128, j])))[0]
            assert y[r, j] == (q - z) * s


def test_blocked_sum_closed_form():
    # X = 1 on group 1 only, q - z = 5 everywhere -> Y[j] = 128 * 5 * s[1][j]
    k, n = 384, 16
    d = int4_inputs(1, k, n, seed=13)
    x = np.zeros((1, k), dtype=np.uint16)
    x[0, 128:256] = 0x3F80
    qw = np.full((k // 8, n), 0x77777777, dtype=np.uint32)
    qz = np.full((k // 128, n // 8), 0x22222222, dtype=np.uint32)
    y = oracle.qgemm_int4(x, qw, d["scales"], qz, 1, k, n)
    s1 = d["scales"][1].view(np.float16).astype(np.float64)
    assert np.array_equal(y[0], 640.0 * s1)


def test_power_of_two_scaling_is_exact():
    d = int4_inputs(2, 256, 16, seed=14)
    y1 = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], 2, 256, 16)
    x2 = f32_to_bf16_bits(oracle.bf16_value(d["x"]) * 4.0)
    y2 = oracle.qgemm_int4(x2, d["qweight"], d["scales"], d["qzeros"], 2, 256, 16)
    np.testing.assert_allclose(y2, 4.0 * y1, rtol=1e-15, atol=0)


def _bf16_py(bits):
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _fp16_py(bits):
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def test_brute_force_small_int4():
    m, k, n = 3, 256, 8
    d = int4_inputs(m, k, n, seed=15)
    y = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    for r in range(m):
        for j in range(n):
            terms = []
            for i in range(k):
                q = (int(d["qweight"][i >> 3, j]) >> ((i & 7) << 2)) & 0xF
                z = (int(d["qzeros"][i >> 7, j >> 3]) >> ((j & 7) << 2)) & 0xF
                s = _fp16_py(d["scales"][i >> 7, j])
                terms.append(_bf16_py(d["x"][r, i]) * ((q - z) * s))
            exact = math.fsum(terms)
            assert abs(y[r, j] - exact) <= 1e-12 * max(1.0, abs(exact))


def test_brute_force_small_int4_without_zero_point():
    m, k, n = 2, 256, 8
    d = int4_inputs(m, k, n, seed=17)
    y = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], None, m, k, n)
    for r in range(m):
        for j in range(n):
            terms = []
            for i in range(k):
                q = (int(d["qweight"][i >> 3, j]) >> ((i & 7) << 2)) & 0xF
                s = _fp16_py(d["scales"][i >> 7, j])
                terms.append(_bf16_py(d["x"][r, i]) * (q * s))
            exact = math.fsum(terms)
            assert abs(y[r, j] - exact) <= 1e-12 * max(1.0, abs(exact))
    part = oracle.qgemm_int4_at(d["x"], d["qweight"], d["scales"], None, k, n, [1], [2, 7])
    np.testing.assert_allclose(part, y[np.ix_([1], [2, 7])], rtol=1e-14, atol=1e-14)


def test_brute_force_small_int4_lora():
    m, k, n, r = 2, 256, 8, 3
    d = int4_inputs(m, k, n, seed=18)
    l = lora_inputs(k, n, r, seed=19, std_a=0.5, std_b=0.5)
    y = oracle.qgemm_int4_lora(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"], l["lora_b"],
                               2.0, m, k, n)
    for row in range(m):
        u = [math.fsum(_bf16_py(d["x"][row, i]) * _bf16_py(l["lora_a"][j, i]) for i in range(k))
             for j in range(r)]
        for col in range(n):
            terms = []
            for i in range(k):
                q = (int(d["qweight"][i >> 3, col]) >> ((i & 7) << 2)) & 0xF
                z = (int(d["qzeros"][i >> 7, col >> 3]) >> ((col & 7) << 2)) & 0xF
                s = _fp16_py(d["scales"][i >> 7, col])
                terms.append(_bf16_py(d["x"][row, i]) * ((q - z) * s))
            terms += [2.0 * u[j] * _bf16_py(l["lora_b"][col, j]) for j in range(r)]
            exact = math.fsum(terms)
            assert abs(y[row, col] - exact) <= 1e-12 * max(1.0, abs(exact))
    part = oracle.qgemm_int4_lora_at(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"],
                                     l["lora_b"], 2.0, k, n, [1], [0, 5])
    np.testing.assert_allclose(part, y[np.ix_([1], [0, 5])], rtol=1e-14, atol=1e-14)


def test_lora_one_hot_closed_form():
    # X = e_0 (one-hot), A = e_j rows, B = ones: the LoRA term is scale * sum_j A[j][0]
    m, k, n, r = 1, 128, 8, 4
    d = int4_inputs(m, k, n, seed=20)
    x = np.zeros((m, k), dtype=np.uint16)
    x[0, 0] = 0x3F80                                   # 1.0
    a = np.zeros((r, k), dtype=np.uint16)
    a[:, 0] = [0x3F80, 0x4000, 0x4040, 0x4080]         # 1, 2, 3, 4
    b = np.full((n, r), 0x3F80, dtype=np.uint16)       # 1.0
    base = oracle.qgemm_int4(x, d["qweight"], d["scales"], d["qzeros"], m, k, n)
    y = oracle.qgemm_int4_lora(x, d["qweight"], d["scales"], d["qzeros"], a, b, 0.5, m, k, n)
    assert np.array_equal(y - base, np.full((m, n), 0.5 * 10.0))


def test_lora_term_exceeds_the_tolerance():
    # at the adapter scale the tests use, the LoRA term moves most outputs by more
    # than the acceptance rule allows: a kernel that dropped it would be rejected
    m, k, n = 8, 1152, 776
    d = int4_inputs(m, k, n, seed=801)
    l = lora_inputs(k, n, 16, seed=802)
    base = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    with_lora = oracle.qgemm_int4_lora(d["x"], d["qweight"], d["scales"], d["qzeros"], l["lora_a"],
                                       l["lora_b"], 2.0, m, k, n)
    assert np.mean(oracle.accept(oracle.round_to_grid(base, "bf16"), with_lora, "bf16")) < 0.2


def test_sampled_outputs_match_full():
    m, k, n = 5, 512, 64
    d = int4_inputs(m, k, n, seed=16)
    full = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    rows, cols = [0, 3, 4], [1, 17, 63]
    part = oracle.qgemm_int4_at(d["x"], d["qweight"], d["scales"], d["qzeros"], k, n, rows, cols)
    np.testing.assert_allclose(part, full[np.ix_(rows, cols)], rtol=1e-14, atol=1e-14)


def test_empty_shapes():
    assert oracle.qgemm_int4(np.zeros((0, 128), np.uint16), np.zeros((16, 8), np.uint32),
                             np.zeros((1, 8), np.uint16), np.zeros((1, 1), np.uint32),
                             0, 128, 8).shape == (0, 8)
    y = oracle.qgemm_int4(np.zeros((2, 0), np.uint16), np.zeros((0, 8), np.uint32),
                          np.zeros((0, 8), np.uint16), np.zeros((0, 1), np.uint32), 2, 0, 8)
    assert y.shape == (2, 8) and np.all(y == 0)


# ----------------------------------------------------------------------------
# the error level of a correct BF16 path, and mistakes the rule must catch
# ----------------------------------------------------------------------------
def _rule():
    with open(os.path.join(GOLDEN, "accuracy_rule.json")) as f:
        return json.load(f)


def test_tolerance_constants_match_the_page():
    rule = _rule()
    assert (oracle.TOL_ABS, oracle.TOL_REL) == (rule["abs"], rule["rel"])


@pytest.fixture(scope="module")
def gemv_case():
    m, k, n = 8, 896, 4864
    d = int4_inputs(m, k, n, seed=17)
    y = oracle.qgemm_int4(d["x"], d["qweight"], d["scales"], d["qzeros"], m, k, n)
    return d, y


def test_correctly_rounded_bf16_sits_at_the_rounding_floor(gemv_case):
    d, y = gemv_case
    rep = oracle.compare(f32_to_bf16_bits(oracle.round_to_grid(y, "bf16")), y, "bf16")
    rule = _rule()
    assert rep["rejected"] == rule["violations"]
    # the page's rms_rel of about 1.66e-3 is the bf16 rounding floor
    assert abs(rep["rms_rel"] - rule["rms_rel_floor"]) < 0.15 * rule["rms_rel_floor"]
    # and the literal bound alone is stricter than bf16's half-ulp for |ref| > ~2
    assert rep["literal_violations"] > 0.01 * rep["n"]


def test_fp32_sequential_accumulation_is_accepted(gemv_case):
    d, y = gemv_case
    m, k, n = 8, 896, 4864
    x = oracle.bf16_value(d["x"]).astype(np.float32)
    w = oracle.dequant(d["qweight"], d["scales"], d["qzeros"], k, n)
    acc = np.zeros((m, n), dtype=np.float32)
    for i in range(k):                      # worst-order fp32 accumulation
        acc += x[:, i:i + 1] * w[i:i + 1, :]
    rep = oracle.compare(f32_to_bf16_bits(acc), y, "bf16")
    assert rep["rejected"] == 0
    big = np.abs(y) >= 1.0          # away from zero, at most one bf16 ulp from RNE(r)
    rep_big = oracle.compare(f32_to_bf16_bits(acc[big]), y[big], "bf16")
    assert rep_big["max_ulp"] <= 1.0


@pytest.mark.parametrize("mistake", ["bf16_weights", "zero_off_by_one", "nibble_order",
                                     "group_shift", "drop_last_group"])
def test_rule_rejects_planted_mistakes(gemv_case, mistake):
    """Plausible kernel bugs, planted in the oracle's own steps on the CPU."""
    d, y = gemv_case
    m, k, n = 8, 896, 4864
    x = oracle.bf16_value(d["x"])
    q = oracle.unpack_qweight(d["qweight"], k, n)
    z = oracle.unpack_qzeros(d["qzeros"], k // 128, n)
    s = oracle.fp16_value(d["scales"])
    g = np.arange(k) // 128
    if mistake == "zero_off_by_one":
        z = z + 1
    if mistake == "nibble_order":
        q = q.reshape(k // 8, 8, n)[:, ::-1, :].reshape(k, n)
    if mistake == "group_shift":
        g = np.minimum((np.arange(k) + 8) // 128, k // 128 - 1)
    w = (q - z[g]) * s[g]
    if mistake == "bf16_weights":
        w = oracle.round_to_grid(w, "bf16")
    if mistake == "drop_last_group":
        w[-128:] = 0
    bad = oracle.round_to_grid(x @ w, "bf16")
    rep = oracle.compare(f32_to_bf16_bits(bad), y, "bf16")
    assert rep["rejected"] > 0.05 * rep["n"], rep


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
    d = dense_inputs(layout, dtype, M, N, K, seed=21, std=1.0)
    c = oracle.dense(layout, dtype, d["a"], d["b"], M, N, K)
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
def test_dense_batched_brute_force(layout):
    bt, M, N, K = 3, 2, 3, 4
    d = dense_batched_inputs(layout, "fp16", bt, M, N, K, seed=24, std=1.0)
    c = oracle.dense_batched(layout, "fp16", d["a"], d["b"], M, N, K)
    assert c.shape == (bt, M, N)
    for q in range(bt):
        for i in range(M):
            for j in range(N):
                terms = []
                for p in range(K):
                    a = d["a"][q, i, p] if layout in ("NT", "NN") else d["a"][q, p, i]
                    b = d["b"][q, j, p] if layout == "NT" else d["b"][q, p, j]
                    terms.append(_fp16_py(a) * _fp16_py(b))
                assert abs(c[q, i, j] - math.fsum(terms)) <= 1e-14 * max(1.0, abs(c[q, i, j]))
    part = oracle.dense_batched_at(layout, "fp16", d["a"], d["b"], 2, [1], [0, 2])
    assert np.array_equal(part, c[2][np.ix_([1], [0, 2])])


def test_dense_batched_scaled_identities():
    # B[q] = (q + 1) I: the products are the A[q] scaled by q + 1, exactly
    bt, M = 4, 8
    d = dense_batched_inputs("NN", "bf16", bt, M, M, M, seed=25, std=1.0)
    eyes = np.stack([_store((q + 1) * np.eye(M), "bf16") for q in range(bt)])
    c = oracle.dense_batched("NN", "bf16", d["a"], eyes, M, M, M)
    for q in range(bt):
        assert np.array_equal(c[q], (q + 1) * oracle.bf16_value(d["a"][q]))


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_dense_identity(layout):
    M = N = K = 16
    d = dense_inputs(layout, "bf16", M, N, K, seed=22, std=1.0)
    eye = _store(np.eye(K), "bf16")
    c = oracle.dense(layout, "bf16", d["a"], eye, M, N, K)
    a = oracle.bf16_value(d["a"])
    assert np.array_equal(c, a if layout != "TN" else a.T)


def test_dense_k1_outer_product_and_1x1x1():
    a = _store([[2.0], [-3.0]], "fp16")                 # A[2][1]
    b = _store([[0.5], [4.0], [1.0]], "fp16")           # B[3][1], NT
    assert oracle.dense("NT", "fp16", a, b, 2, 3, 1).tolist() == [[1.0, 8.0, 2.0],
                                                                  [-1.5, -12.0, -3.0]]
    one = _store([[1.5]], "bf16")
    assert oracle.dense("TN", "bf16", one, one, 1, 1, 1).tolist() == [[2.25]]


def test_fp32_decoder_matches_struct_unpack():
    # special values, subnormals, extremes and a seeded sample of all patterns
    rng = np.random.default_rng(3)
    pats = np.concatenate([
        np.array([0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x3F800000, 0xBF800000, 0x7F7FFFFF,
                  0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x33800000], dtype=np.uint64),
        rng.integers(0, 2 ** 32, size=20000, dtype=np.uint64)]).astype(np.uint32)
    got = oracle.fp32_value(pats)
    for b, g in zip(pats.tolist(), got.tolist()):
        want = struct.unpack("<f", struct.pack("<I", b))[0]
        if math.isnan(want):
            assert math.isnan(g)
        else:
            assert g == want, (hex(b), g, want)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
def test_dense_fp32_brute_force(layout):
    M, N, K = 3, 4, 6
    d = dense_inputs(layout, "fp32", M, N, K, seed=26, std=1.0)
    c = oracle.dense(layout, "fp32", d["a"], d["b"], M, N, K)
    absd = oracle.dense_absdot(layout, "fp32", d["a"], d["b"])
    dec = lambda v: struct.unpack("<f", struct.pack("<I", int(v)))[0]
    for i in range(M):
        for j in range(N):
            terms = []
            for p in range(K):
                a = d["a"][i, p] if layout in ("NT", "NN") else d["a"][p, i]
                b = d["b"][j, p] if layout == "NT" else d["b"][p, j]
                terms.append(dec(a) * dec(b))
            assert abs(c[i, j] - math.fsum(terms)) <= 1e-14 * max(1.0, abs(c[i, j]))
            assert abs(absd[i, j] - math.fsum(abs(t) for t in terms)) <= 1e-14 * absd[i, j]


def test_fp32_bound_accepts_fp32_sums_and_rejects_a_dropped_term():
    M, N, K = 16, 16, 2048
    d = dense_inputs("NT", "fp32", M, N, K, seed=27, std=1.0)
    r = oracle.dense("NT", "fp32", d["a"], d["b"], M, N, K)
    absd = oracle.dense_absdot("NT", "fp32", d["a"], d["b"])
    a = oracle.fp32_value(d["a"]).astype(np.float32)
    b = oracle.fp32_value(d["b"]).astype(np.float32)
    # a plain sequential fp32 evaluation lies inside the bound
    y = np.zeros((M, N), dtype=np.float32)
    for p in range(K):
        y = (y + np.outer(a[:, p], b[:, p]).astype(np.float32)).astype(np.float32)
    rep = oracle.compare_fp32(y.view(np.uint32), r, absd, K)
    assert rep["rejected"] == 0 and rep["rms_rel"] < 2e-5, rep
    # a dropped k slice (8 of 2048 terms, the size of one lane's step) is outside it
    y2 = (y - (a[:, 64:72].astype(np.float64) @ b[:, 64:72].T.astype(np.float64))).astype(np.float32)
    rep2 = oracle.compare_fp32(y2.view(np.uint32), r, absd, K)
    assert rep2["rejected"] > 0.9 * M * N, rep2


def test_dense_fp16_subnormals_are_kept():
    a = np.array([[0x0001, 0x03FF]], dtype=np.uint16)       # 2^-24, largest subnormal
    b = np.array([[0x3C00], [0x4000]], dtype=np.uint16)     # [K][N] = [1; 2]
    c = oracle.dense("NN", "fp16", a, b, 1, 1, 2)
    assert c[0, 0] == 2.0 ** -24 + 2 * (1023 / 1024) * 2.0 ** -14


def test_dense_dropped_k_slice_is_rejected():
    M, N, K = 64, 64, 256
    d = dense_inputs("NT", "bf16", M, N, K, seed=23)
    c = oracle.dense("NT", "bf16", d["a"], d["b"], M, N, K)
    a = oracle.bf16_value(d["a"]).copy()
    a[:, 32:64] = 0                                         # a lost 32-wide K slice
    bad = oracle.round_to_grid(a @ oracle.bf16_value(d["b"]).T, "bf16")
    rep = oracle.compare(f32_to_bf16_bits(bad), c, "bf16")
    assert rep["rms_rel"] > 0.05


def test_row_sumsq_closed_forms_and_brute_force():
    # constant rows: n c^2 exactly (c = 1.5 and -0.25 are bf16 values)
    y = np.zeros((2, 40), dtype=np.uint16)
    y[0, :] = 0x3FC0          # 1.5
    y[1, :] = 0xBE80          # -0.25
    r = oracle.row_sumsq(y)
    assert r[0] == 40 * 2.25 and r[1] == 40 * 0.0625
    # brute force with math.fsum over struct-decoded values, random bf16 rows
    import math
    import struct

    from qgemm_inputs import f32_to_bf16_bits

    rng = np.random.default_rng(5)
    bits = f32_to_bf16_bits((rng.normal(size=(3, 77)) * 3.0).astype(np.float32))
    for i in range(3):
        vals = [struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits[i]]
        exact = math.fsum(v * v for v in vals)
        assert abs(oracle.row_sumsq(bits[i:i + 1])[0] - exact) <= 1e-14 * exact   # fp64 sum order
    # the bound covers a sequential fp32 sum, and rejects a dropped term
    v = oracle.bf16_value(bits).astype(np.float32)
    seq = np.zeros(3, dtype=np.float32)
    for j in range(77):
        seq = (seq + v[:, j] * v[:, j]).astype(np.float32)
    assert np.all(np.abs(seq - oracle.row_sumsq(bits)) <= oracle.row_sumsq_bound(bits))
    dropped = oracle.row_sumsq(bits[:, 1:])
    big = np.abs(oracle.bf16_value(bits[:, 0])) ** 2 > oracle.row_sumsq_bound(bits)
    assert np.all(np.abs(dropped - oracle.row_sumsq(bits))[big] > oracle.row_sumsq_bound(bits)[big])
