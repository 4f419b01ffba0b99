"""Pins for the oracle's 2-bit threshold quantizer with error feedback.

Everything here checks the oracle against what the MXNet PR #8342 page
("[WIP] 2bit gradient compression") fixes -- the printed worked example, the
rule's inclusive comparisons, the format -- or against mathematics: brute
force over code patterns with an independent bit-string builder, residual
sign and error bounds, error-feedback telescoping, and special cases.
"""
import itertools
import json
import struct

import numpy as np
import pytest

import oracle
import synthetic_inputs as si


def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def bits_f32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(u)))[0]


def ulp32(x: np.ndarray) -> np.ndarray:
    x = np.abs(np.asarray(x, dtype=np.float32))
    return (np.nextafter(x, np.float32(np.inf), dtype=np.float32) - x).astype(np.float64)


# ---------------------------------------------------------------- golden ----

def test_worked_example_matches_printed_block(golden_dir):
    ex = json.loads((golden_dir / "worked_example_2bit.json").read_text())
    g = np.array(ex["constructed_grad"], dtype=np.float32)
    r = np.array(ex["constructed_residual"], dtype=np.float32)
    compr = oracle.quantize_2bit(g, r, ex["neg_threshold"], ex["pos_threshold"])

    printed = ex["printed_compr"]
    assert compr.size == len(printed) == 4
    # Header: thresholds and the original size, as fp32.
    assert bits_f32(compr[0]) == printed[0]
    assert bits_f32(compr[1]) == printed[1]
    assert bits_f32(compr[2]) == float(printed[2]) == ex["n"]
    # The packed element, read as fp32, equals the printed value to the
    # printed 8 significant digits ...
    got = bits_f32(compr[3])
    assert float(f"{got:.7e}") == printed[3]
    # ... and its bit pattern is the printed bit string.
    assert int(ex["printed_last_element_bits"].replace(" ", ""), 2) == int(compr[3])


def test_worked_example_residual_and_dequantized(golden_dir):
    ex = json.loads((golden_dir / "worked_example_2bit.json").read_text())
    g = np.array(ex["constructed_grad"], dtype=np.float32)
    r = np.zeros(8, dtype=np.float32)
    compr = oracle.quantize_2bit(g, r, -2.0, 2.0)
    deq = oracle.dequantize_2bit(compr, 8)
    # Codes 00 01 00 10 01 00 00 10: the printed bit string.
    np.testing.assert_array_equal(deq, [0, 2, 0, -2, 2, 0, 0, -2])
    # Residual carries what was not sent: g - deq (all exact here).
    np.testing.assert_array_equal(r, g - deq)


# ---------------------------------------------------------- brute force ----

def _bitstring_words(codes_per_segment, offset, seg_words):
    """Independent builder: write each code as two characters, MSB-first,
    into a '0'/'1' string of seg_words*32 characters, then parse."""
    pair = {0: "00", 1: "01", 2: "10"}
    out = []
    for codes in codes_per_segment:
        chars = ["00"] * (16 * seg_words)
        for k, c in enumerate(codes):
            chars[offset + k] = pair[c]
        s = "".join(chars)
        out.extend(int(s[32 * w:32 * (w + 1)], 2) for w in range(seg_words))
    return out


@pytest.mark.parametrize("k", range(1, 10))
def test_packing_every_code_pattern_every_offset(k):
    """All 3^k code patterns of length k <= 9, starting at each of the 16
    in-word offsets (so patterns also straddle a word boundary)."""
    patterns = list(itertools.product((0, 1, 2), repeat=k))
    value = {0: np.float32(0.25), 1: np.float32(0.75), 2: np.float32(-0.75)}
    offsets = range(16) if k <= 6 else (0, 7, 9, 15)
    seg_words = 2
    seg = 16 * seg_words
    for off in offsets:
        g = np.zeros(len(patterns) * seg, dtype=np.float32)
        for p, codes in enumerate(patterns):
            for j, c in enumerate(codes):
                g[p * seg + off + j] = value[c]
        r = np.zeros_like(g)
        compr = oracle.quantize_2bit(g, r, -0.5, 0.5)
        expect = _bitstring_words(patterns, off, seg_words)
        assert compr[3:].tolist() == expect, f"k={k} offset={off}"


@pytest.mark.parametrize("n", [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 4095, 4096, 4097])
def test_format_size_and_tail(n):
    g = si.normal_f32(7, n, 1.0)
    r = np.zeros(n, dtype=np.float32)
    compr = oracle.quantize_2bit(g, r, -0.5, 0.5)
    assert compr.size == 3 + (n + 15) // 16 == oracle.compressed_2bit_words(n)
    assert bits_f32(compr[2]) == float(n)
    if n % 16:
        used = n % 16
        # codes past the end are 00: the low 2*(16-used) bits are zero
        assert int(compr[-1]) & ((1 << (2 * (16 - used))) - 1) == 0


# ------------------------------------------------------ classification ----

@pytest.mark.parametrize("thr", [0.5, 0.01, 0.005, 2.0, 1e-30, 3.4e38])
def test_threshold_edges_inclusive(thr):
    pos = np.float32(thr)
    neg = np.float32(-thr)
    up = np.nextafter(pos, np.float32(np.inf))
    dn = np.nextafter(pos, np.float32(0))
    v = np.array([pos, up, dn, neg, -up, -dn, 0.0, -0.0], dtype=np.float32)
    r = np.zeros_like(v)
    compr = oracle.quantize_2bit(v, r, neg, pos)
    deq = oracle.dequantize_2bit(compr, v.size)
    # at or beyond a threshold -> that threshold; strictly inside -> 0
    np.testing.assert_array_equal(deq, np.array([pos, pos, 0, neg, neg, 0, 0, 0], np.float32))


def test_ieee_special_values():
    """NaN, infinities, FLT_MAX, subnormals and signed zeros go through the
    inclusive comparisons of [MX] "Two bit quantization" as IEEE fixes them:
    a NaN compares false both ways (code 00, residual NaN); an infinity is
    beyond either threshold and stays infinite; FLT_MAX - 0.5 rounds back to
    FLT_MAX; subnormals are kept (no flush to zero); -0 + 0 is +0."""
    tiny = bits_f32(1)  # 2^-149
    fmax = np.finfo(np.float32).max
    g = np.array([np.nan, np.inf, -np.inf, fmax, -fmax, tiny, -tiny, 0.0, -0.0, 0.5, -0.5],
                 np.float32)
    r = np.zeros_like(g)
    compr = oracle.quantize_2bit(g, r, -0.5, 0.5)
    np.testing.assert_array_equal(
        oracle.dequantize_2bit(compr, g.size),
        np.array([0, 0.5, -0.5, 0.5, -0.5, 0, 0, 0, 0, 0.5, -0.5], np.float32))
    assert np.isnan(r[0])
    np.testing.assert_array_equal(
        r[1:].view(np.uint32),
        np.array([0x7F800000, 0xFF800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x00000001, 0x80000001,
                  0, 0, 0, 0], np.uint32))


def test_subnormal_thresholds():
    """Thresholds of 3 * 2^-149 and values k * 2^-149: every operation is exact
    on subnormals, so the codes and residuals are those of integer
    arithmetic on k (in units of 2^-149)."""
    unit = lambda m: (m if m >= 0 else 0x80000000 | -m) if m != 0 else 0  # noqa: E731
    ks = list(range(-5, 6))
    g = np.array([bits_f32(unit(k)) for k in ks], np.float32)
    t = np.float32(bits_f32(3))
    r = np.zeros_like(g)
    compr = oracle.quantize_2bit(g, r, -t, t)
    deq = oracle.dequantize_2bit(compr, g.size)
    code = [1 if k >= 3 else 2 if k <= -3 else 0 for k in ks]
    np.testing.assert_array_equal(deq.view(np.uint32),
                                  np.array([unit({0: 0, 1: 3, 2: -3}[c]) for c in code],
                                           np.uint32))
    np.testing.assert_array_equal(
        r.view(np.uint32),
        np.array([unit(k - {0: 0, 1: 3, 2: -3}[c]) for k, c in zip(ks, code)], np.uint32))
    # the residual carries: 2 + 1 units reach the threshold exactly
    g2 = np.array([bits_f32(2)] * 3, np.float32)
    r2 = np.array([bits_f32(1), 0.0, bits_f32(0x80000001)], np.float32)
    deq2 = oracle.dequantize_2bit(oracle.quantize_2bit(g2, r2, -t, t), 3)
    np.testing.assert_array_equal(deq2.view(np.uint32), np.array([3, 0, 0], np.uint32))
    np.testing.assert_array_equal(r2.view(np.uint32), np.array([0, 2, 1], np.uint32))


def test_unused_code_11_dequantizes_to_zero():
    compr = np.array([f32_bits(-1.0), f32_bits(1.0), f32_bits(16.0), 0xFFFFFFFF], np.uint32)
    np.testing.assert_array_equal(oracle.dequantize_2bit(compr, 16), np.zeros(16, np.float32))


# ------------------------------------------------------------- residual ----

@pytest.mark.parametrize("sigma,thr", [(0.5, 0.5), (0.01, 0.01), (0.005, 0.005), (0.03, 0.01)])
def test_residual_invariants(sigma, thr):
    n = 200_000
    rng_r = si.normal_f32(99, n, sigma)
    g = si.normal_f32(5, n, sigma)
    r = rng_r.copy()
    v = (g + rng_r).astype(np.float32)  # the carried value, one fp32 add
    compr = oracle.quantize_2bit(g, r, -thr, thr)
    d = oracle.dequantize_2bit(compr, n)
    pos, neg = np.float32(thr), np.float32(-thr)
    z = d == 0
    # code 00: strictly inside, residual is v bit for bit
    assert np.all((v[z] > neg) & (v[z] < pos))
    np.testing.assert_array_equal(r[z].view(np.uint32), v[z].view(np.uint32))
    # code 01 / 10: residual keeps the sign of the excess
    assert np.all(r[d == pos] >= 0) and np.all(v[d == pos] >= pos)
    assert np.all(r[d == neg] <= 0) and np.all(v[d == neg] <= neg)
    # deq + residual == grad + old residual, up to one rounding of v - d
    err = np.abs(d.astype(np.float64) + r.astype(np.float64) - v.astype(np.float64))
    assert np.all(err <= 0.5 * ulp32(r))


def test_error_feedback_telescopes():
    """Over T iterations: sum_t deq_t + r_T == sum_t g_t, up to the
    roundings of the two fp32 operations per iteration."""
    n, T, thr = 100_000, 10, 0.5
    r = np.zeros(n, dtype=np.float32)
    sum_g = np.zeros(n)
    sum_d = np.zeros(n)
    bound = np.zeros(n)
    for t in range(T):
        g = si.normal_f32(si.grad_seed(0, t), n, 0.5)
        v = (g + r).astype(np.float32)
        compr = oracle.quantize_2bit(g, r, -thr, thr)
        d = oracle.dequantize_2bit(compr, n)
        sum_g += g
        sum_d += d
        bound += 0.5 * ulp32(v) + 0.5 * ulp32(r)
    assert np.all(np.abs(sum_d + r - sum_g) <= bound)


def test_huge_thresholds_send_nothing():
    n = 10_000
    g = si.normal_f32(3, n, 1.0)
    r0 = si.normal_f32(4, n, 1.0)
    r = r0.copy()
    fmax = np.finfo(np.float32).max
    compr = oracle.quantize_2bit(g, r, -fmax, fmax)
    assert np.all(compr[3:] == 0)
    np.testing.assert_array_equal(r, (g + r0).astype(np.float32))


# ------------------------------------------------------------ W-sum ----

def test_sum_of_one_worker_is_dequantize():
    n = 5000
    g = si.normal_f32(11, n, 0.5)
    compr = oracle.quantize_2bit(g, np.zeros(n, np.float32), -0.5, 0.5)
    np.testing.assert_array_equal(oracle.dequantize_2bit_sum([compr], n),
                                  oracle.dequantize_2bit(compr, n))


def test_sum_dyadic_thresholds_is_exact():
    """With thresholds +-0.5 every partial sum of <= 8 terms is exact in
    fp32, so the W-sum equals the exact (fp64) sum of the dequantized parts."""
    n, W = 20_000, 8
    comprs, deqs = [], []
    for w in range(W):
        g = si.normal_f32(si.grad_seed(w, 0), n, 0.5)
        c = oracle.quantize_2bit(g, np.zeros(n, np.float32), -0.5, 0.5)
        comprs.append(c)
        deqs.append(oracle.dequantize_2bit(c, n).astype(np.float64))
    exact = np.sum(deqs, axis=0)
    np.testing.assert_array_equal(oracle.dequantize_2bit_sum(comprs, n).astype(np.float64), exact)


def test_sum_order_is_worker_order():
    """Different thresholds per worker: the result is the left-to-right fp32
    sum (worker 0 first), and within W-1 roundings of the exact sum."""
    n, W = 20_000, 5
    thr = [0.3, 0.01, 0.7, 1e-3, 0.11]
    comprs, deqs = [], []
    for w in range(W):
        g = si.normal_f32(si.grad_seed(w, 3), n, 0.5)
        c = oracle.quantize_2bit(g, np.zeros(n, np.float32), -thr[w], thr[w])
        comprs.append(c)
        deqs.append(oracle.dequantize_2bit(c, n))
    got = oracle.dequantize_2bit_sum(comprs, n)
    acc = deqs[0].copy()
    for w in range(1, W):
        acc = (acc + deqs[w]).astype(np.float32)
    np.testing.assert_array_equal(got, acc)
    exact = np.sum([d.astype(np.float64) for d in deqs], axis=0)
    mag = np.sum([np.abs(d.astype(np.float64)) for d in deqs], axis=0)
    assert np.all(np.abs(got - exact) <= (W - 1) * 2.0 ** -24 * mag)


# ------------------------------------------------------ randomised ----

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None, derandomize=True, database=None)
@given(n=st.integers(0, 3000), neg=st.floats(1e-6, 100.0), pos=st.floats(1e-6, 100.0),
       sigma=st.floats(1e-6, 100.0), seed=st.integers(0, 2 ** 32 - 1))
def test_residual_invariants_random_asymmetric(n, neg, pos, sigma, seed):
    g = si.normal_f32(seed, n, sigma)
    r0 = si.normal_f32(seed ^ 0x5A5A, n, sigma)
    r = r0.copy()
    v = (g + r0).astype(np.float32)
    neg32, pos32 = np.float32(-neg), np.float32(pos)
    compr = oracle.quantize_2bit(g, r, neg32, pos32)
    assert compr.size == 3 + (n + 15) // 16
    d = oracle.dequantize_2bit(compr, n)
    up, dn = v >= pos32, v <= neg32
    np.testing.assert_array_equal(d, np.where(up, pos32, np.where(dn, neg32, np.float32(0))))
    np.testing.assert_array_equal(r[~up & ~dn].view(np.uint32), v[~up & ~dn].view(np.uint32))
    assert np.all(r[up] >= 0) and np.all(r[dn] <= 0)
    err = np.abs(d.astype(np.float64) + r.astype(np.float64) - v.astype(np.float64))
    assert np.all(err <= 0.5 * ulp32(r))
