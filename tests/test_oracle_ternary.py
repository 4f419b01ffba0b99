"""Pins for the oracle's dense ternary packing (five codes per byte): the
optimization the MXNet PR #8342 page ("Two bit quantization") leaves for
later, because a three-valued code wastes one of its two bits.

The error-feedback arithmetic is the 2-bit quantizer's, so the first pin is
equivalence with the (already pinned) 2-bit oracle: same residual bits, same
dequantized values, same W-sums. The packing is pinned by brute force over
digit patterns against an independent base-3 builder, and by the format's
size and byte-range properties.
"""
import itertools

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synthetic_inputs as si


@pytest.mark.parametrize("n", [0, 1, 4, 5, 6, 19, 20, 21, 39, 40, 41, 4096, 100_003])
def test_size_formula_and_byte_range(n):
    g = si.normal_f32(n, n, 1.0)
    c = oracle.quantize_ternary(g, np.zeros(n, np.float32), -0.5, 0.5)
    nbytes = (n + 4) // 5
    assert c.size == 3 + (nbytes + 3) // 4 == oracle.compressed_ternary_words(n)
    payload = c[3:].view(np.uint8)
    assert np.all(payload[:nbytes] <= 242)
    assert np.all(payload[nbytes:] == 0)
    assert c[0] == np.float32(-0.5).view(np.uint32) and c[1] == np.float32(0.5).view(np.uint32)
    assert c[2] == np.float32(n).view(np.uint32)


@pytest.mark.parametrize("sigma,neg,pos", [(0.5, -0.5, 0.5), (0.01, -0.01, 0.01),
                                           (1.0, -0.3, 1.7), (0.05, -2.0, 0.001)])
def test_equivalent_to_2bit(sigma, neg, pos):
    n = 50_003
    g = si.normal_f32(3, n, sigma)
    r0 = si.normal_f32(4, n, sigma)
    r2, r3 = r0.copy(), r0.copy()
    c2 = oracle.quantize_2bit(g, r2, neg, pos)
    c3 = oracle.quantize_ternary(g, r3, neg, pos)
    np.testing.assert_array_equal(r2.view(np.uint32), r3.view(np.uint32))
    np.testing.assert_array_equal(oracle.dequantize_ternary(c3, n), oracle.dequantize_2bit(c2, n))


def test_sum_equivalent_to_2bit():
    n, W = 20_001, 7
    c2s, c3s = [], []
    for w in range(W):
        g = si.normal_f32(si.grad_seed(w, 1), n, 0.3)
        thr = 0.1 + 0.05 * w
        c2s.append(oracle.quantize_2bit(g, np.zeros(n, np.float32), -thr, thr))
        c3s.append(oracle.quantize_ternary(g, np.zeros(n, np.float32), -thr, thr))
    np.testing.assert_array_equal(oracle.dequantize_ternary_sum(c3s, n),
                                  oracle.dequantize_2bit_sum(c2s, n))


@pytest.mark.parametrize("k", range(1, 8))
def test_packing_every_pattern(k):
    """All 3^k digit patterns of length k <= 7 at each of the 5 in-byte
    offsets (so longer patterns straddle bytes), against bytes built from
    base-3 digit strings with int(s, 3)."""
    patterns = list(itertools.product((0, 1, 2), repeat=k))
    value = {0: np.float32(0.25), 1: np.float32(0.75), 2: np.float32(-0.75)}
    seg = 15  # three bytes per pattern
    for off in range(5):
        g = np.zeros(len(patterns) * seg, np.float32)
        for p, codes in enumerate(patterns):
            for j, c in enumerate(codes):
                g[p * seg + off + j] = value[c]
        comp = oracle.quantize_ternary(g, np.zeros_like(g), -0.5, 0.5)
        got = comp[3:].view(np.uint8)[:len(patterns) * 3]
        expect = []
        for codes in patterns:
            digits = ["0"] * seg
            for j, c in enumerate(codes):
                digits[off + j] = str(c)
            expect += [int("".join(digits[5 * b:5 * b + 5]), 3) for b in range(3)]
        assert got.tolist() == expect, (k, off)


def test_decode_of_every_byte_value():
    """Bytes 0..255 in one block: digits are read by repeated division by 3
    (independently here with divmod), and a leading digit of 3 (bytes 243 and
    up, never written) is an unused code that dequantizes to 0."""
    n = 256 * 5
    c = np.zeros(oracle.compressed_ternary_words(n), np.uint32)
    c[0], c[1] = np.float32(-1.0).view(np.uint32), np.float32(2.0).view(np.uint32)
    c[2] = np.float32(n).view(np.uint32)
    c[3:].view(np.uint8)[:256] = np.arange(256, dtype=np.uint8)
    out = oracle.dequantize_ternary(c, n)
    val = {0: 0.0, 1: 2.0, 2: -1.0}
    for b in range(256):
        rest, digs = b, []
        for _ in range(4):
            rest, d = divmod(rest, 3)
            digs.append(d)
        lead = rest  # 0..3
        expect = [val.get(lead, 0.0)] + [val[d] for d in reversed(digs)]
        assert out[5 * b:5 * b + 5].tolist() == expect, b


@settings(max_examples=40, deadline=None, derandomize=True, database=None)
@given(n=st.integers(0, 3000), neg=st.floats(1e-5, 10.0), pos=st.floats(1e-5, 10.0),
       seed=st.integers(0, 2 ** 32 - 1))
def test_equivalent_to_2bit_random(n, neg, pos, seed):
    g = si.normal_f32(seed, n, 1.0)
    r2, r3 = np.zeros(n, np.float32), np.zeros(n, np.float32)
    c2 = oracle.quantize_2bit(g, r2, -neg, pos)
    c3 = oracle.quantize_ternary(g, r3, -neg, pos)
    np.testing.assert_array_equal(r2.view(np.uint32), r3.view(np.uint32))
    np.testing.assert_array_equal(oracle.dequantize_ternary(c3, n), oracle.dequantize_2bit(c2, n))
