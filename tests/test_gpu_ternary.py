"""GPU parity of the dense ternary packing (five codes per byte) against the
oracle, through the C ABI. Words and residuals bit for bit; dequantized sums
within 1e-6 relative error (bit-exact in fact: same fp32 operations in the
same order).

Workloads: ragged sizes around every element (20 values) and tile (1280
values) boundary, 16-byte-aligned and 4-byte-misaligned; the small
error-feedback case (4096 values ~ N(0, 0.5^2), thresholds +-0.5, 10
iterations); threshold edges; dequantize-and-sum for W up to 64 (compile-time
and run-time worker counts); every byte value 0..255 (the never-written bytes
243..255 included); and the ResNet-50-sized flat gradient (25,557,032 values
~ N(0, 0.01^2), thresholds +-0.01, W = 8 workers x 3 iterations, then the
W = 8 dequantize-and-sum) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

SIZES = [0, 1, 2, 3, 4, 5, 6, 19, 20, 21, 39, 40, 41, 63, 64, 65, 1279, 1280, 1281,
         1300, 2559, 2560, 2561, 5119, 5120, 5121, 5141, 65536 + 7, (1 << 20) + 3]


def gpu_compress(gcq, g_np, r_np, neg, pos, misalign=False):
    n = g_np.size
    g = gu.dev(g_np, misalign)
    r = gu.dev(r_np, misalign)
    compr = gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32, misalign=misalign, fill=-1)
    gcq.compress_ternary(g, r, neg, pos, compr)
    gu.sync()
    return gu.host(compr, np.uint32), gu.host(r)


@pytest.mark.parametrize("n", [0, 1, 20, 21, 1280, 25_557_032, 2 ** 33 + 5])
def test_sizes_match_oracle(gcq, n):
    assert gcq.gc_compressed_ternary_words(n) == 3 + (n + 19) // 20
    if n < 10 ** 8:
        assert gcq.gc_compressed_ternary_words(n) == oracle.compressed_ternary_words(n)


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("n", SIZES)
def test_ragged_sizes(gcq, n, misalign):
    announce(f"ternary compress n={n} misalign={misalign}")
    g = si.normal_f32(5000 + n, n, 0.5)
    r0 = si.normal_f32(6000 + n, n, 0.25)
    compr, r_gpu = gpu_compress(gcq, g, r0.copy(), -0.5, 0.5, misalign)
    r_or = r0.copy()
    c_or = oracle.quantize_ternary(g, r_or, -0.5, 0.5)
    np.testing.assert_array_equal(compr, c_or)
    np.testing.assert_array_equal(r_gpu.view(np.uint32), r_or.view(np.uint32))
    c_dev = gu.dev(c_or)
    base = si.normal_f32(7000 + n, n, 1.0)
    out = gu.dev(base, misalign)
    gcq.decompress_ternary(c_dev, n, out, accumulate=True)
    out2 = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    gcq.decompress_ternary(c_dev, n, out2)
    gu.sync()
    d_or = oracle.dequantize_ternary(c_or, n)
    np.testing.assert_array_equal(gu.host(out2), d_or)
    np.testing.assert_array_equal(gu.host(out), (base + d_or).astype(np.float32))


def test_small_error_feedback_10_iterations(gcq):
    announce("ternary n=4096 sigma=0.5 thr=0.5 x10 iterations")
    n = 4096
    g_dev = gu.empty(n, torch.float32)
    r_dev = torch.zeros(n, dtype=torch.float32, device=gu.DEV)
    compr = gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32, fill=-1)
    r_or = np.zeros(n, np.float32)
    for t in range(10):
        g = si.normal_f32(si.grad_seed(0, t), n, 0.5)
        g_dev.copy_(torch.from_numpy(g))
        gcq.compress_ternary(g_dev, r_dev, -0.5, 0.5, compr)
        c_or = oracle.quantize_ternary(g, r_or, -0.5, 0.5)
        gu.sync()
        np.testing.assert_array_equal(gu.host(compr, np.uint32), c_or, err_msg=f"iter {t}")
        np.testing.assert_array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32))


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("kind", ["specials", "subnormal"])
def test_ieee_specials_and_subnormals(gcq, kind, misalign):
    """NaN, infinities, FLT_MAX, subnormals and signed zeros among the values,
    or values and thresholds that are all multiples of 2^-149."""
    n = 5141
    announce(f"ternary IEEE edge case {kind} misalign={misalign}")
    if kind == "specials":
        g, r0, t = si.with_ieee_specials(31, n, 0.01), si.normal_f32(32, n, 0.005), np.float32(0.01)
    else:
        g, r0, t = si.subnormal_units(33, n, 9), si.subnormal_units(34, n, 4), np.float32(2.0 ** -147)
    compr, r_gpu = gpu_compress(gcq, g, r0, -t, t, misalign)
    r_or = r0.copy()
    c_or = oracle.quantize_ternary(g, r_or, -t, t)
    np.testing.assert_array_equal(compr, c_or)
    nan = np.isnan(r_or)
    np.testing.assert_array_equal(np.isnan(r_gpu), nan)
    np.testing.assert_array_equal(r_gpu[~nan].view(np.uint32), r_or[~nan].view(np.uint32))
    out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    gcq.decompress_ternary_sum([gu.dev(c_or)] * 3, n, out)
    gu.sync()
    np.testing.assert_array_equal(gu.host(out).view(np.uint32),
                                  oracle.dequantize_ternary_sum([c_or] * 3, n).view(np.uint32))


@pytest.mark.parametrize("thr", [0.5, 0.01, 2.0, 1e-30])
def test_threshold_edges(gcq, thr):
    announce(f"ternary threshold edges thr={thr}")
    pos = np.float32(thr)
    up = np.nextafter(pos, np.float32(np.inf))
    dn = np.nextafter(pos, np.float32(0))
    v = np.array([pos, up, dn, -pos, -up, -dn, 0.0, -0.0] * 200, np.float32)
    compr, r_gpu = gpu_compress(gcq, v, np.zeros_like(v), -pos, pos)
    r_or = np.zeros_like(v)
    np.testing.assert_array_equal(compr, oracle.quantize_ternary(v, r_or, -pos, pos))
    np.testing.assert_array_equal(r_gpu.view(np.uint32), r_or.view(np.uint32))


def test_every_byte_value_decodes_like_the_oracle(gcq):
    """A block whose payload holds each byte 0..255 (so also the bytes
    243..255 that compress never writes), repeated to span several tiles."""
    announce("ternary decode of all 256 byte values")
    reps = 40
    n = 256 * 5 * reps
    c = np.zeros(oracle.compressed_ternary_words(n), np.uint32)
    c[0], c[1] = np.float32(-0.75).view(np.uint32), np.float32(1.25).view(np.uint32)
    c[2] = np.float32(n).view(np.uint32)
    c[3:].view(np.uint8)[:256 * reps] = np.tile(np.arange(256, dtype=np.uint8), reps)
    expect = oracle.dequantize_ternary(c, n)
    for misalign in (False, True):
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.decompress_ternary(gu.dev(c), n, out)
        gu.sync()
        np.testing.assert_array_equal(gu.host(out), expect)


@pytest.mark.parametrize("W", [1, 2, 3, 8, 9, 13, 16, 17, 33, 64])
@pytest.mark.parametrize("n", [1, 17, 1000, 1281, 5121, 100_003])
def test_dequantize_sum(gcq, W, n):
    announce(f"ternary dequantize-sum W={W} n={n}")
    comprs = []
    for w in range(W):
        thr = 0.05 + 0.01 * (w % 7)
        g = si.normal_f32(si.grad_seed(w, 9), n, 0.05)
        comprs.append(oracle.quantize_ternary(g, np.zeros(n, np.float32), -thr, 1.5 * thr))
    expect = oracle.dequantize_ternary_sum(comprs, n)
    for misalign in (False, True):
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.decompress_ternary_sum([gu.dev(c) for c in comprs], n, out)
        gu.sync()
        got = gu.host(out)
        assert np.all(np.abs(got - expect) <= 1e-6 * np.abs(expect))
        np.testing.assert_array_equal(got, expect)  # same order -> bit-exact


def test_same_residuals_and_values_as_2bit_on_gpu(gcq):
    """The two packings share the arithmetic: on the GPU too, the residuals
    match bit for bit and the dequantized W-sums are identical."""
    announce("ternary vs 2-bit on the GPU, W=4 n=300007")
    n, W = 300_007, 4
    c3, c2 = [], []
    for w in range(W):
        g = gu.dev(si.normal_f32(si.grad_seed(w, 3), n, 0.1))
        r3 = torch.zeros(n, dtype=torch.float32, device=gu.DEV)
        r2 = torch.zeros(n, dtype=torch.float32, device=gu.DEV)
        c3.append(gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32))
        c2.append(gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32))
        gcq.compress_ternary(g, r3, -0.08, 0.08, c3[-1])
        gcq.compress_2bit(g, r2, -0.08, 0.08, c2[-1])
        gu.sync()
        assert torch.equal(r3.view(torch.int32), r2.view(torch.int32)), w
    o3 = gu.empty(n, torch.float32)
    o2 = gu.empty(n, torch.float32)
    gcq.decompress_ternary_sum(c3, n, o3)
    gcq.decompress_2bit_sum(c2, n, o2)
    gu.sync()
    assert torch.equal(o3.view(torch.int32), o2.view(torch.int32))


@pytest.mark.slow
def test_resnet50_flat_gradient_full_size(gcq):
    """25,557,032 values, W = 8 workers x 3 error-feedback iterations, then
    the W = 8 dequantize-and-sum."""
    n, W, T, thr = si.RESNET50_PARAMS, 8, 3, 0.01
    words = gcq.gc_compressed_ternary_words(n)
    g_dev = gu.empty(n, torch.float32)
    r_dev = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for _ in range(W)]
    c_dev = [gu.empty(words, torch.int32) for _ in range(W)]
    r_or = [np.zeros(n, np.float32) for _ in range(W)]
    c_or = [None] * W
    for t in range(T):
        for w in range(W):
            announce(f"ternary full size n={n} iter={t} worker={w}")
            g = si.normal_f32(si.grad_seed(w, t), n, 0.01)
            g_dev.copy_(torch.from_numpy(g))
            c_dev[w].fill_(-1)
            gcq.compress_ternary(g_dev, r_dev[w], -thr, thr, c_dev[w])
            c_or[w] = oracle.quantize_ternary(g, r_or[w], -thr, thr)
            gu.sync()
            assert np.array_equal(gu.host(c_dev[w], np.uint32), c_or[w]), (t, w)
            assert np.array_equal(gu.host(r_dev[w]).view(np.uint32), r_or[w].view(np.uint32)), (t, w)
    announce("ternary full size dequantize-sum W=8")
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.decompress_ternary_sum(c_dev, n, out)
    gu.sync()
    got = gu.host(out)
    expect = oracle.dequantize_ternary_sum(c_or, n)
    assert np.all(np.abs(got - expect) <= 1e-6 * np.abs(expect))
    assert np.array_equal(got, expect)
    # one more iteration of worker 0 and the sum with the gradient, residual
    # and output 4 bytes off 16-byte alignment (the 4-byte-access kernels at
    # full size)
    announce("ternary full size, buffers 4 bytes off alignment")
    g = si.normal_f32(si.grad_seed(0, T), n, 0.01)
    r_mis = gu.dev(r_or[0], True)
    gcq.compress_ternary(gu.dev(g, True), r_mis, -thr, thr, c_dev[0])
    c_or[0] = oracle.quantize_ternary(g, r_or[0], -thr, thr)
    out_mis = gu.empty(n, torch.float32, misalign=True, fill=float("nan"))
    gcq.decompress_ternary_sum(c_dev, n, out_mis)
    gu.sync()
    assert np.array_equal(gu.host(c_dev[0], np.uint32), c_or[0])
    assert np.array_equal(gu.host(r_mis).view(np.uint32), r_or[0].view(np.uint32))
    assert np.array_equal(gu.host(out_mis), oracle.dequantize_ternary_sum(c_or, n))
