"""Pins for the oracle's QSGD max-norm quantizer and the GlobalRandK draw.

Sources: the vineeths96 "Gradient-Compression" page ("Quantization for
Distributed Optimization": QSGDMaxNorm is all-reduce compatible, so workers
share one max-norm and their integer levels can be summed; GRandK-MN uses
K = 10000 shared indices). The level is floor(|g|/norm * s + u) with u
uniform in [0, 1).

Pins: the level function against exact rational floor on a grid; closed-form
cases (|g| = norm gives s, g = 0 gives 0, integral x is deterministic);
unbiasedness over many seeds; library routines for max and sum; exact
rationals for dequantization; uniformity of the rand-K draw over all ordered
pairs for a tiny n; distinctness and range at full size.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import stats

import oracle
import synthetic_inputs as si


def _f32(x):
    return np.float32(x)


# ------------------------------------------------------ level function ----

def _x_grid(s):
    xs = {0.0, float(s), 1e-45, 1e-38, 2.0 ** -30, 2.0 ** -25, 0.5, 1.0 - 2 ** -24}
    for k in range(s + 1):
        xs.add(float(k))
        xs.add(float(np.nextafter(_f32(k), _f32(np.inf))))
        xs.add(float(np.nextafter(_f32(k), _f32(0))))
    rng = np.random.default_rng(0)
    xs.update(float(v) for v in (rng.random(300) * s).astype(np.float32))
    return sorted(v for v in xs if 0.0 <= v <= s)


def _u_grid():
    ks = {0, 1, 2, 2 ** 23, 2 ** 24 - 2, 2 ** 24 - 1, 3 * 2 ** 21}
    rng = np.random.default_rng(1)
    ks.update(int(k) for k in rng.integers(0, 2 ** 24, 40))
    return sorted(ks)


@pytest.mark.parametrize("s", [1, 7, 127])
def test_stochastic_level_is_exact_floor(s):
    for x in _x_grid(s):
        fx = Fraction(float(_f32(x)))
        frac = fx - (fx.numerator // fx.denominator)
        # u values that land x + u exactly on the next integer, and around it
        special = set()
        if frac:
            k_hit = (1 - frac) * 2 ** 24
            if k_hit.denominator == 1:
                special.update({int(k_hit) - 1, int(k_hit), int(k_hit) + 1})
        for k in _u_grid() + sorted(v for v in special if 0 <= v < 2 ** 24):
            u = k * 2.0 ** -24
            expect = (fx + Fraction(k, 2 ** 24)).__floor__()
            assert oracle.stochastic_level(x, u) == expect, (x, k)


def test_uniform24_endpoints_and_exactness():
    assert oracle.uniform24(0) == 0.0
    assert oracle.uniform24(0xFF) == 0.0
    assert oracle.uniform24(0x100) == 2.0 ** -24
    assert oracle.uniform24(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    rng = np.random.default_rng(2)
    for r in rng.integers(0, 2 ** 32, 1000):
        assert oracle.uniform24(int(r)) == (int(r) >> 8) / 2 ** 24


# ------------------------------------------------------ closed forms ----

@pytest.mark.parametrize("s", [1, 7, 127])
def test_norm_element_maps_to_plus_minus_s(s):
    g = si.normal_f32(3, 1000, 0.02)
    j = int(np.argmax(np.abs(g)))
    norm = oracle.maxnorm([g])
    for seed in range(20):
        q = oracle.qsgd_quantize(g, norm, s, seed, 0)
        assert q[j] == (s if g[j] > 0 else -s)
        assert np.all(np.abs(q.astype(np.int32)) <= s)


def test_zero_and_negative_zero_give_zero():
    g = np.array([0.0, -0.0, 0.0, -0.0, 1.0], dtype=np.float32)
    for seed in range(50):
        q = oracle.qsgd_quantize(g, 1.0, 127, seed, 3)
        assert q[:4].tolist() == [0, 0, 0, 0]


def test_zero_norm_gives_zero_levels():
    g = np.zeros(100, np.float32)
    assert np.all(oracle.qsgd_quantize(g, 0.0, 127, 0, 0) == 0)


def test_integral_x_is_deterministic():
    """norm = 1, s = 4, g = j/4: x = j exactly, so the level is j for every u."""
    j = np.arange(-4, 5)
    g = (j / 4).astype(np.float32)
    for seed in range(100):
        np.testing.assert_array_equal(oracle.qsgd_quantize(g, 1.0, 4, seed, 1), j)


def test_level_brackets_scaled_value_and_keeps_sign():
    n, s = 50_000, 127
    g = si.heavy_tailed_f32(4, n, 0.02)
    norm = oracle.maxnorm([g])
    q = oracle.qsgd_quantize(g, norm, s, 9, 2).astype(np.int64)
    x = (np.abs(g) / norm).astype(np.float32) * np.float32(s)
    lo = np.floor(x.astype(np.float64))
    m = np.abs(q)
    assert np.all((m == lo) | (m == lo + 1))
    assert np.all(m[x == lo] == lo[x == lo])
    assert np.all(np.sign(q)[m > 0] == np.sign(g)[m > 0])


def test_level_uses_word_index_mod_4_of_block_index_div_4():
    """Composition of the oracle's own steps: element i draws word i % 4 of
    Philox(counter = (i/4, 0, worker, 0), key = seed)."""
    n, s, seed, worker = 64, 127, 0x1234_5678_9ABC, 5
    g = si.normal_f32(8, n, 1.0)
    norm = oracle.maxnorm([g])
    q = oracle.qsgd_quantize(g, norm, s, seed, worker)
    for i in range(n):
        r = oracle.philox4x32_10([i // 4, 0, worker, 0], [seed & 0xFFFFFFFF, seed >> 32])[i % 4]
        x = np.float32(np.float32(abs(g[i]) / norm) * np.float32(s))
        m = oracle.stochastic_level(x, oracle.uniform24(int(r)))
        assert q[i] == (-m if g[i] < 0 else m)


def test_quantize_at_matches_quantize():
    n = 10_001
    g = si.normal_f32(12, n, 0.01)
    norm = oracle.maxnorm([g])
    full = oracle.qsgd_quantize(g, norm, 127, 77, 6)
    idx = np.array([0, 1, 2, 3, 4, 5000, 9999, 10000], dtype=np.uint64)
    np.testing.assert_array_equal(
        oracle.qsgd_quantize_at(g[idx.astype(np.int64)], idx, norm, 127, 77, 6),
        full[idx.astype(np.int64)])


# ---------------------------------------------------------- unbiased ----

def test_unbiased_over_seeds():
    """E[q] * norm / s == g: mean over 10^4 seeds within 6 binomial sigmas
    (plus the 2^-24-level bias bound of a 24-bit u)."""
    n, s, M = 64, 7, 10_000
    g = si.normal_f32(21, n, 1.0)
    norm = oracle.maxnorm([g])
    acc = np.zeros(n)
    for seed in range(M):
        acc += oracle.qsgd_quantize(g, norm, s, seed, 0)
    mean = acc / M * float(norm) / s
    x = (np.abs(g) / norm).astype(np.float32) * np.float32(s)
    p = x.astype(np.float64) - np.floor(x)
    sigma = np.sqrt(p * (1 - p) / M) * float(norm) / s
    tol = 6 * sigma + 2.0 ** -24 * float(norm) / s + 1e-7 * np.abs(g)
    assert np.all(np.abs(mean - g.astype(np.float64)) <= tol)


def test_level_up_frequency_matches_fraction():
    """For one element with fractional part p the level-up frequency over
    seeds is p (exactly floor(p*2^24)/2^24 for a 24-bit u)."""
    s, M = 1, 20_000
    g = np.array([0.3, 1.0, 0.71, 0.05], dtype=np.float32)  # norm = 1
    ups = np.zeros(4)
    for seed in range(M):
        ups += oracle.qsgd_quantize(g, 1.0, s, seed, 4) == 1
    p = np.floor(g.astype(np.float64) * 2 ** 24) / 2 ** 24
    p[1] = 1.0
    for k in (0, 2, 3):
        bt = stats.binomtest(int(ups[k]), M, p[k])
        assert bt.pvalue > 1e-6, (k, ups[k] / M, p[k])
    assert ups[1] == M


# ---------------------------------------------------- norm, sum, deq ----

def test_maxnorm_matches_numpy():
    W, n = 8, 30_001
    gs = [si.heavy_tailed_f32(si.grad_seed(w, 0), n, 0.02) for w in range(W)]
    gs[3][17] = np.float32(-7.5)  # the largest magnitude is negative
    expect = np.max(np.abs(np.stack(gs)))
    assert oracle.maxnorm(gs) == expect == np.float32(7.5)
    tiny = [np.array([1e-45, -0.0], np.float32)]
    assert oracle.maxnorm(tiny) == np.float32(1e-45)


def test_level_sum_matches_numpy():
    W, n = 8, 10_000
    rng = np.random.default_rng(5)
    qs = [rng.integers(-127, 128, n).astype(np.int8) for _ in range(W)]
    np.testing.assert_array_equal(oracle.level_sum(qs),
                                  np.sum(np.stack(qs).astype(np.int64), axis=0))


@pytest.mark.parametrize("s", [7, 127])
def test_dequantize_within_two_roundings(s):
    rng = np.random.default_rng(6)
    S = rng.integers(-8 * s, 8 * s + 1, 5000).astype(np.int32)
    S[:3] = [0, s, -s]
    norm = np.float32(0.8234567)
    out = oracle.qsgd_dequantize(S, norm, s)
    assert out[0] == 0.0
    for k in range(S.size):
        exact = Fraction(float(norm)) * int(S[k]) / s
        err = abs(Fraction(float(out[k])) - exact)
        assert err <= abs(exact) * Fraction(1, 2 ** 23), (k, int(S[k]))


def _round_f32(x: Fraction) -> Fraction:
    """x rounded to the nearest binary32 value, ties to even (normal range
    and zero; the values below stay far from overflow and underflow)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp                      # in [2^23, 2^24)
    q, r = divmod(m.numerator, m.denominator)
    twice = 2 * r
    if twice > m.denominator or (twice == m.denominator and q % 2 == 1):
        q += 1
    return sign * q * ulp


def test_round_f32_helper_matches_numpy_on_doubles():
    """The rounding helper agrees with numpy's (correctly rounded) float64 ->
    float32 conversion, halfway cases included."""
    rng = np.random.default_rng(61)
    xs = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-20, 20, 2000))
    # exact halfway points between neighbouring binary32 values, both parities
    for m in (1, 2, 3, 1 << 22, (1 << 23) - 1):
        xs += [(2 ** 23 + m + 0.5) * 2.0 ** -23, -(2 ** 23 + m + 0.5) * 2.0 ** -30]
    for x in xs:
        assert _round_f32(Fraction(x)) == Fraction(float(np.float32(x))), x


@pytest.mark.parametrize("s", [7, 127])
def test_dequantize_is_the_product_rounded_then_the_quotient_rounded(s):
    """out = fl(fl(norm * S) / s), from exact rationals: each step rounded
    once to binary32 in that order. The other order, fl(norm * fl(S / s)),
    differs on some of these inputs, so the check tells the two apart."""
    rng = np.random.default_rng(60 + s)
    S = rng.integers(-8 * s, 8 * s + 1, 3000).astype(np.int32)
    norms = [np.float32(v) for v in (0.8234567, 3.0e-3, 17.25, 1.1e-7)]
    other_order_differs = False
    for norm in norms:
        out = oracle.qsgd_dequantize(S, norm, s)
        fn = Fraction(float(norm))
        for k in range(S.size):
            want = _round_f32(_round_f32(fn * int(S[k])) / s)
            assert Fraction(float(out[k])) == want, (float(norm), int(S[k]))
            alt = _round_f32(fn * _round_f32(Fraction(int(S[k]), s)))
            other_order_differs |= alt != want
    assert other_order_differs


# ----------------------------------------------------------- rand-K ----

def test_randk_tiny_uniform_over_ordered_pairs():
    n, K, M = 5, 2, 100_000
    counts = np.zeros((n, n), dtype=np.int64)
    for seed in range(M):
        a, b = oracle.randk_indices(n, K, seed)
        counts[a, b] += 1
    assert np.all(np.diag(counts) == 0)
    obs = counts[~np.eye(n, dtype=bool)]
    assert obs.size == 20
    assert stats.chisquare(obs).pvalue > 1e-6


def test_randk_first_index_uniform():
    n, M = 7, 70_000
    first = np.array([oracle.randk_indices(n, 1, seed)[0] for seed in range(M)])
    assert stats.chisquare(np.bincount(first, minlength=n)).pvalue > 1e-6


@pytest.mark.parametrize("n,K", [(1, 1), (16, 16), (1000, 1000), (1000, 10), (1 << 20, 10_000),
                                 (si.RESNET50_PARAMS, 10_000)])
def test_randk_distinct_in_range(n, K):
    idx = oracle.randk_indices(n, K, 42)
    assert idx.size == K
    assert len(np.unique(idx)) == K
    assert int(idx.max()) < n
    if K == n:
        np.testing.assert_array_equal(np.sort(idx), np.arange(n))


def test_randk_prefix_property():
    """Fewer draws give the prefix of more draws (step i uses only draw i)."""
    a = oracle.randk_indices(100_000, 500, 9)
    b = oracle.randk_indices(100_000, 2000, 9)
    np.testing.assert_array_equal(a, b[:500])


@pytest.mark.parametrize("n,K,seed", [(1, 1, 0), (2, 2, 5), (7, 7, 11), (50, 13, 12345),
                                      (300, 300, 2 ** 40 + 7), (1000, 37, 2 ** 63 + 1)])
def test_randk_matches_an_explicit_fisher_yates(n, K, seed):
    """The draw's definition restated with Python integers and a list:
    step i draws j = i + floor(R (n - i) / 2^64) from Philox words (w0, w1)
    of counter (i, 0, 0, 1), swaps positions i and j, and takes the value now
    at position i. A consistency check of the C arithmetic (the 128-bit
    product, 32-bit counters, 64-bit seeds split into the key), not an
    independent pin: the uniformity tests above are those."""
    perm = list(range(n))
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for i in range(K):
        w = oracle.philox4x32_10([i, 0, 0, 1], key)
        R = (int(w[1]) << 32) | int(w[0])
        j = i + ((R * (n - i)) >> 64)
        perm[i], perm[j] = perm[j], perm[i]
    np.testing.assert_array_equal(oracle.randk_indices(n, K, seed),
                                  np.array(perm[:K], dtype=np.uint32))


def test_randk_rejects_k_above_n():
    with pytest.raises(ValueError):
        oracle.randk_indices(10, 11, 0)
    assert oracle.randk_indices(10, 0, 0).size == 0


def test_gather_scatter_match_numpy():
    x = si.normal_f32(1, 1000, 1.0)
    idx = oracle.randk_indices(1000, 100, 3)
    np.testing.assert_array_equal(oracle.gather(x, idx), x[idx])
    dense = oracle.scatter_dense(x[:100], idx, 1000)
    expect = np.zeros(1000, np.float32)
    expect[idx] = x[:100]
    np.testing.assert_array_equal(dense, expect)


# ------------------------------------------------------ randomised ----

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=60, deadline=None, derandomize=True, database=None)
@given(n=st.integers(1, 50_000), frac=st.floats(0.0, 1.0), seed=st.integers(0, 2 ** 64 - 1))
def test_randk_random_shapes(n, frac, seed):
    K = int(frac * n)
    idx = oracle.randk_indices(n, K, seed)
    assert idx.size == K and len(np.unique(idx)) == K
    assert K == 0 or int(idx.max()) < n
    if K > 1:
        np.testing.assert_array_equal(oracle.randk_indices(n, K // 2, seed), idx[:K // 2])


@settings(max_examples=60, deadline=None, derandomize=True, database=None)
@given(n=st.integers(1, 5000), s=st.integers(1, 127), scale=st.floats(1e-30, 1e30),
       seed=st.integers(0, 2 ** 64 - 1), worker=st.integers(0, 2 ** 32 - 1))
def test_levels_bracket_random(n, s, scale, seed, worker):
    g = (si.normal_f32(seed % (2 ** 32), n, 1.0) * np.float32(scale)).astype(np.float32)
    g = g[np.isfinite(g)]
    if g.size == 0:
        return
    norm = oracle.maxnorm([g])
    q = oracle.qsgd_quantize(g, norm, s, seed, worker).astype(np.int64)
    if norm == 0:
        assert np.all(q == 0)
        return
    x = (np.abs(g) / norm).astype(np.float32) * np.float32(s)
    lo = np.floor(x.astype(np.float64))
    m = np.abs(q)
    assert np.all((m == lo) | (m == lo + 1)) and np.all(m <= s)
    assert np.all(np.sign(q)[m > 0] == np.sign(g)[m > 0])
