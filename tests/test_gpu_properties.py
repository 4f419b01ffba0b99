"""Randomised GPU parity against the oracle (hypothesis, derandomised so a
run is reproducible): sizes across tile and word boundaries, asymmetric
thresholds, misaligned buffers, worker counts, level counts and seeds."""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st, HealthCheck

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

SETTINGS = settings(max_examples=40, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


@SETTINGS
@given(n=st.integers(0, 70_000), neg=st.floats(1e-4, 4.0), pos=st.floats(1e-4, 4.0),
       sigma=st.floats(1e-3, 8.0), misalign=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_compress_decompress_random(gcq, n, neg, pos, sigma, misalign, seed):
    announce(f"prop compress n={n} neg=-{neg} pos={pos} sigma={sigma} mis={misalign} seed={seed}")
    g = si.normal_f32(seed, n, sigma)
    r0 = si.normal_f32(seed + 1, n, sigma / 2)
    neg32, pos32 = np.float32(-neg), np.float32(pos)
    g_dev, r_dev = gu.dev(g, misalign), gu.dev(r0, misalign)
    compr = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, misalign=misalign, fill=-1)
    gcq.compress_2bit(g_dev, r_dev, float(neg32), float(pos32), compr)
    out = gu.empty(n, torch.float32, misalign=not misalign, fill=float("nan"))
    gcq.decompress_2bit(compr, n, out)
    gu.sync()
    r_or = r0.copy()
    c_or = oracle.quantize_2bit(g, r_or, neg32, pos32)
    np.testing.assert_array_equal(gu.host(compr, np.uint32), c_or)
    np.testing.assert_array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32))
    np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit(c_or, n))


@SETTINGS
@given(n=st.integers(0, 70_000), neg=st.floats(1e-4, 4.0), pos=st.floats(1e-4, 4.0),
       sigma=st.floats(1e-3, 8.0), misalign=st.booleans(), W=st.integers(1, 10),
       seed=st.integers(0, 2 ** 31 - 1))
def test_ternary_random(gcq, n, neg, pos, sigma, misalign, W, seed):
    announce(f"prop ternary n={n} neg=-{neg} pos={pos} sigma={sigma} mis={misalign} W={W} seed={seed}")
    neg32, pos32 = np.float32(-neg), np.float32(pos)
    comprs_or, comprs_dev = [], []
    for w in range(W):
        g = si.normal_f32(seed + 31 * w, n, sigma)
        r0 = si.normal_f32(seed + 31 * w + 1, n, sigma / 2)
        r_dev = gu.dev(r0, misalign)
        compr = gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32, misalign=misalign, fill=-1)
        gcq.compress_ternary(gu.dev(g, misalign), r_dev, float(neg32), float(pos32), compr)
        r_or = r0.copy()
        c_or = oracle.quantize_ternary(g, r_or, neg32, pos32)
        gu.sync()
        np.testing.assert_array_equal(gu.host(compr, np.uint32), c_or)
        np.testing.assert_array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32))
        comprs_or.append(c_or)
        comprs_dev.append(compr)
    out = gu.empty(n, torch.float32, misalign=not misalign, fill=float("nan"))
    gcq.decompress_ternary_sum(comprs_dev, n, out)
    gu.sync()
    np.testing.assert_array_equal(gu.host(out), oracle.dequantize_ternary_sum(comprs_or, n))


@SETTINGS
@given(W=st.integers(1, 12), n=st.integers(1, 40_000), seed=st.integers(0, 2 ** 31 - 1))
def test_dequantize_sum_random(gcq, W, n, seed):
    announce(f"prop dequantize-sum W={W} n={n} seed={seed}")
    rng = np.random.default_rng(seed)
    comprs = []
    for w in range(W):
        neg, pos = np.float32(-rng.uniform(0.01, 1.0)), np.float32(rng.uniform(0.01, 1.0))
        g = si.normal_f32(seed + 17 * w, n, 0.5)
        comprs.append(oracle.quantize_2bit(g, np.zeros(n, np.float32), neg, pos))
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.decompress_2bit_sum([gu.dev(c) for c in comprs], n, out)
    gu.sync()
    np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit_sum(comprs, n))


@SETTINGS
@given(W=st.integers(1, 10), n=st.integers(1, 30_000), s=st.integers(1, 127),
       scale=st.sampled_from([1e-3, 0.02, 1.0, 50.0]), misalign=st.booleans(),
       seed=st.integers(0, 2 ** 63 - 1))
def test_qsgd_step_random(gcq, W, n, s, scale, misalign, seed):
    announce(f"prop qsgd W={W} n={n} s={s} scale={scale} mis={misalign} seed={seed}")
    grads = [si.heavy_tailed_f32((seed + w) % (2 ** 32), n, scale) for w in range(W)]
    g_dev = [gu.dev(g, misalign) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    levels = [gu.empty(n, torch.int8, misalign=misalign) for _ in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, levels[w])
    sums = gu.empty(n, torch.int32)
    out = gu.empty(n, torch.float32)
    gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)
    gu.sync()
    norm_or = oracle.maxnorm(grads)
    assert np.float32(gu.host(norm)[0]).view(np.uint32) == norm_or.view(np.uint32)
    lv_or = [oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(grads)]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w])
    s_or = oracle.level_sum(lv_or)
    np.testing.assert_array_equal(gu.host(sums), s_or)
    np.testing.assert_array_equal(gu.host(out), oracle.qsgd_dequantize(s_or, norm_or, s))


@SETTINGS
@given(W=st.integers(1, 10), n=st.integers(1, 30_000), s=st.integers(1, 127),
       scale=st.sampled_from([1e-3, 0.02, 1.0, 50.0]), misalign=st.booleans(),
       with_sums=st.booleans(), seed=st.integers(0, 2 ** 63 - 1))
def test_qsgd_fused_random(gcq, W, n, s, scale, misalign, with_sums, seed):
    announce(f"prop qsgd fused W={W} n={n} s={s} scale={scale} mis={misalign} sums={with_sums} seed={seed}")
    grads = [si.heavy_tailed_f32((seed + 3 * w) % (2 ** 32), n, scale) for w in range(W)]
    g_dev = [gu.dev(g, misalign) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    sums = gu.empty(n, torch.int32, misalign=misalign) if with_sums else None
    out = gu.empty(n, torch.float32, misalign=not misalign)
    gcq.qsgd_quantize_sum(g_dev, norm, s, seed, out, sums=sums)
    gu.sync()
    norm_or = oracle.maxnorm(grads)
    s_or = oracle.level_sum([oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(grads)])
    if with_sums:
        np.testing.assert_array_equal(gu.host(sums), s_or)
    np.testing.assert_array_equal(gu.host(out), oracle.qsgd_dequantize(s_or, norm_or, s))


@SETTINGS
@given(n=st.integers(1, 200_000), frac=st.floats(0.0, 1.0), seed=st.integers(0, 2 ** 63 - 1))
def test_grandk_indices_random(gcq, n, frac, seed):
    K = min(n, int(frac * min(n, 30_000)))
    announce(f"prop grandk n={n} K={K} seed={seed}")
    idx = gu.empty(max(K, 1), torch.int32, fill=-1)
    ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_indices(n, K, seed, idx[:K], ws)
    gu.sync()
    np.testing.assert_array_equal(gu.host(idx, np.uint32)[:K], oracle.randk_indices(n, K, seed))


@SETTINGS
@given(n=st.integers(1, 150_000), frac=st.floats(0.0, 1.0), W=st.integers(1, 12),
       s=st.integers(1, 127), misalign=st.booleans(), seed=st.integers(0, 2 ** 63 - 1))
def test_grandk_mn_step_random(gcq, n, frac, W, s, misalign, seed):
    K = min(n, int(frac * min(n, 24_000)))
    announce(f"prop grandk_mn_step n={n} K={K} W={W} s={s} mis={misalign} seed={seed}")
    grads = [si.normal_f32((seed + 7 * w) % (2 ** 32), n, 0.01) for w in range(W)]
    idx = gu.empty(max(K, 1), torch.int32, fill=-1)
    sums = gu.empty(max(K, 1), torch.int32, fill=-1)
    dense = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_mn_step([gu.dev(g) for g in grads], K, seed, s, idx, dense, ws, sums=sums)
    gu.sync()
    idx_or = oracle.randk_indices(n, K, seed)
    gk = [oracle.gather(g, idx_or) for g in grads]
    nrm = oracle.maxnorm(gk) if K > 0 else np.float32(0.0)
    S = oracle.level_sum([oracle.qsgd_quantize(g, nrm, s, seed, w) for w, g in enumerate(gk)])
    np.testing.assert_array_equal(gu.host(idx, np.uint32)[:K], idx_or)
    np.testing.assert_array_equal(gu.host(sums)[:K], S)
    np.testing.assert_array_equal(gu.host(dense),
                                  oracle.scatter_dense(oracle.qsgd_dequantize(S, nrm, s), idx_or, n))
