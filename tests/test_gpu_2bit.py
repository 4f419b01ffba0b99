"""GPU parity of the 2-bit error-feedback path against the oracle.

The HIP library is called through its C ABI (the ctypes binding) on device
buffers; the oracle runs on the same input bytes on the CPU. Packed words and
residuals must match bit for bit; dequantized sums within 1e-6 relative error
(they are in fact bit-exact: same fp32 operations in the same order).

Workloads: the page's worked example (thresholds +-2, 8 values); the small
error-feedback case (4096 values ~ N(0, 0.5^2), thresholds +-0.5, 10
iterations with fresh gradients, seeds 0..9); ragged sizes around every tile
boundary, 16-byte-aligned and 4-byte-misaligned; the ResNet-50-sized flat
gradient (25,557,032 values ~ N(0, 0.01^2), thresholds +-0.01, 5 iterations,
then the W = 8 dequantize-and-sum) in the launch configuration the benchmark
times; and the BERT-Base parameter list through the many-tensor launcher
(198 tensors, 109,482,240 values ~ N(0, 0.005^2), thresholds +-0.005, 3
iterations).
"""
import json

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

SIZES = [0, 1, 2, 3, 4, 5, 15, 16, 17, 31, 63, 64, 65, 255, 256, 257, 1023, 1024, 1025,
         4095, 4096, 4097, 4111, 8191, 65536 + 7, (1 << 20) + 3]


def gpu_compress(gcq, g_np, r_np, neg, pos, misalign=False, poison=True):
    n = g_np.size
    g = gu.dev(g_np, misalign)
    r = gu.dev(r_np, misalign)
    words = gcq.gc_compressed_2bit_words(n)
    compr = gu.empty(words, torch.int32, misalign=misalign, fill=-1 if poison else None)
    gcq.compress_2bit(g, r, neg, pos, compr)
    gu.sync()
    return gu.host(compr, np.uint32), gu.host(r)


def test_worked_example(gcq, golden_dir):
    announce("2-bit worked example")
    ex = json.loads((golden_dir / "worked_example_2bit.json").read_text())
    g = np.array(ex["constructed_grad"], np.float32)
    r = np.zeros(8, np.float32)
    compr, r_gpu = gpu_compress(gcq, g, r, ex["neg_threshold"], ex["pos_threshold"])
    r_or = np.zeros(8, np.float32)
    compr_or = oracle.quantize_2bit(g, r_or, ex["neg_threshold"], ex["pos_threshold"])
    assert compr.tolist() == compr_or.tolist()
    assert int(compr[3]) == int(ex["printed_last_element_bits"].replace(" ", ""), 2)
    np.testing.assert_array_equal(r_gpu.view(np.uint32), r_or.view(np.uint32))


def test_small_error_feedback_10_iterations(gcq):
    announce("2-bit n=4096 sigma=0.5 thr=0.5 x10 iterations")
    n = 4096
    g_dev = gu.empty(n, torch.float32)
    r_dev = torch.zeros(n, dtype=torch.float32, device=gu.DEV)
    compr = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1)
    r_or = np.zeros(n, np.float32)
    for t in range(10):
        g = si.normal_f32(si.grad_seed(0, t), n, 0.5)
        g_dev.copy_(torch.from_numpy(g))
        gcq.compress_2bit(g_dev, r_dev, -0.5, 0.5, compr)
        c_or = oracle.quantize_2bit(g, r_or, -0.5, 0.5)
        gu.sync()
        np.testing.assert_array_equal(gu.host(compr, np.uint32), c_or, err_msg=f"iter {t}")
        np.testing.assert_array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32))
        out = gu.empty(n, torch.float32, fill=float("nan"))
        gcq.decompress_2bit(compr, n, out)
        gu.sync()
        np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit(c_or, n))


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("n", SIZES)
def test_ragged_sizes(gcq, n, misalign):
    announce(f"2-bit compress n={n} misalign={misalign}")
    g = si.normal_f32(1000 + n, n, 0.5)
    r0 = si.normal_f32(2000 + n, n, 0.25)
    compr, r_gpu = gpu_compress(gcq, g, r0.copy(), -0.5, 0.5, misalign)
    r_or = r0.copy()
    c_or = oracle.quantize_2bit(g, r_or, -0.5, 0.5)
    np.testing.assert_array_equal(compr, c_or)
    np.testing.assert_array_equal(r_gpu.view(np.uint32), r_or.view(np.uint32))
    # decompress (overwrite and accumulate) into aligned and misaligned outputs
    c_dev = gu.dev(c_or)
    base = si.normal_f32(3000 + n, n, 1.0)
    out = gu.dev(base, misalign)
    gcq.decompress_2bit(c_dev, n, out, accumulate=True)
    out2 = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    gcq.decompress_2bit(c_dev, n, out2)
    gu.sync()
    d_or = oracle.dequantize_2bit(c_or, n)
    np.testing.assert_array_equal(gu.host(out2), d_or)
    np.testing.assert_array_equal(gu.host(out), (base + d_or).astype(np.float32))


@pytest.mark.parametrize("thr", [0.5, 0.01, 2.0, 1e-30])
def test_threshold_edges(gcq, thr):
    announce(f"2-bit threshold edges thr={thr}")
    pos = np.float32(thr)
    up = np.nextafter(pos, np.float32(np.inf))
    dn = np.nextafter(pos, np.float32(0))
    v = np.array([pos, up, dn, -pos, -up, -dn, 0.0, -0.0] * 9, np.float32)
    compr, r_gpu = gpu_compress(gcq, v, np.zeros_like(v), -pos, pos)
    r_or = np.zeros_like(v)
    np.testing.assert_array_equal(compr, oracle.quantize_2bit(v, r_or, -pos, pos))
    np.testing.assert_array_equal(r_gpu.view(np.uint32), r_or.view(np.uint32))


def ieee_case(kind: str, n: int):
    """Gradient, starting residual and thresholds of an IEEE edge case:
    'specials' puts NaN, infinities, FLT_MAX, subnormals and signed zeros
    among N(0, 0.01^2) values (thresholds +-0.01); 'subnormal' uses values,
    residuals and thresholds that are all multiples of 2^-149."""
    if kind == "specials":
        return (si.with_ieee_specials(21, n, 0.01), si.normal_f32(22, n, 0.005),
                np.float32(0.01))
    return si.subnormal_units(23, n, 9), si.subnormal_units(24, n, 4), np.float32(2.0 ** -147)


def assert_residuals_match(r_gpu, r_or):
    """Bit for bit, except that NaN must meet NaN (payloads are not compared)."""
    nan = np.isnan(r_or)
    np.testing.assert_array_equal(np.isnan(r_gpu), nan)
    np.testing.assert_array_equal(r_gpu[~nan].view(np.uint32), r_or[~nan].view(np.uint32))


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("kind", ["specials", "subnormal"])
def test_ieee_specials_and_subnormals(gcq, kind, misalign):
    n = 4099
    announce(f"2-bit IEEE edge case {kind} misalign={misalign}")
    g, r0, t = ieee_case(kind, n)
    compr, r_gpu = gpu_compress(gcq, g, r0, -t, t, misalign)
    r_or = r0.copy()
    c_or = oracle.quantize_2bit(g, r_or, -t, t)
    np.testing.assert_array_equal(compr, c_or)
    assert_residuals_match(r_gpu, r_or)
    # the blocks decode and sum like the oracle's (subnormal thresholds included)
    blocks = [c_or, oracle.quantize_2bit(g, r_or.copy(), -t, t), c_or]
    out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    gcq.decompress_2bit_sum([gu.dev(c) for c in blocks], n, out)
    gu.sync()
    np.testing.assert_array_equal(gu.host(out).view(np.uint32),
                                  oracle.dequantize_2bit_sum(blocks, n).view(np.uint32))


def test_workers_on_concurrent_streams(gcq):
    """The workers' compresses run on two streams at once and the sum on a
    third that waits for both; two error-feedback iterations, the second
    ordered after the first sum. The calls share no state, so the results
    are the oracle's."""
    n, W, thr = 1_000_003, 6, 0.05
    announce(f"2-bit EF on concurrent streams W={W} n={n}")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    sum_stream = torch.cuda.Stream()
    grads = [si.normal_f32(si.grad_seed(w, 70), n, 0.05) for w in range(W)]
    g_dev = [gu.dev(g) for g in grads]
    r_dev = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for _ in range(W)]
    c_dev = [gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1) for _ in range(W)]
    out = gu.empty(n, torch.float32, fill=float("nan"))
    r_or = [np.zeros(n, np.float32) for _ in range(W)]
    gu.sync()
    for it in range(2):
        for w in range(W):
            gcq.compress_2bit(g_dev[w], r_dev[w], -thr, thr, c_dev[w], stream=streams[w % 2])
        for st in streams:
            sum_stream.wait_stream(st)
        gcq.decompress_2bit_sum(c_dev, n, out, stream=sum_stream)
        for st in streams:  # the next compresses overwrite what the sum reads
            st.wait_stream(sum_stream)
        c_or = [oracle.quantize_2bit(grads[w], r_or[w], -thr, thr) for w in range(W)]
    gu.sync()
    for w in range(W):
        np.testing.assert_array_equal(gu.host(c_dev[w], np.uint32), c_or[w])
        np.testing.assert_array_equal(gu.host(r_dev[w]).view(np.uint32), r_or[w].view(np.uint32))
    np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit_sum(c_or, n))


@pytest.mark.parametrize("W", [1, 2, 3, 8, 9, 13, 16, 17, 33, 64])
@pytest.mark.parametrize("n", [1, 17, 1000, 4097, 100_003])
def test_dequantize_sum(gcq, W, n):
    announce(f"2-bit dequantize-sum W={W} n={n}")
    comprs = []
    for w in range(W):
        thr = 0.05 + 0.01 * (w % 7)
        g = si.normal_f32(si.grad_seed(w, 7), n, 0.05)
        comprs.append(oracle.quantize_2bit(g, np.zeros(n, np.float32), -thr, thr))
    expect = oracle.dequantize_2bit_sum(comprs, n)
    for misalign in (False, True):
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.decompress_2bit_sum([gu.dev(c) for c in comprs], n, out)
        gu.sync()
        got = gu.host(out)
        assert np.all(np.abs(got - expect) <= 1e-6 * np.abs(expect))
        np.testing.assert_array_equal(got, expect)  # same order -> bit-exact


@pytest.mark.parametrize("W", [1, 3, 8])
@pytest.mark.parametrize("n", [16, 1000, 4097, 100_003])
def test_dequantize_arbitrary_words(gcq, W, n):
    """Blocks whose words hold random bits: every 2-bit pattern occurs,
    including 11, which the compressor never writes and which decodes to 0,
    and the bits past n in the last word are not zero (they must be
    ignored)."""
    announce(f"2-bit dequantize of arbitrary words W={W} n={n}")
    rng = np.random.default_rng(131 * n + W)
    comprs = []
    for w in range(W):
        c = rng.integers(0, 2 ** 32, oracle.compressed_2bit_words(n), dtype=np.uint64).astype(np.uint32)
        c[0] = np.float32(-0.25 - 0.01 * w).view(np.uint32)
        c[1] = np.float32(0.5 + 0.01 * w).view(np.uint32)
        c[2] = np.float32(n).view(np.uint32)
        comprs.append(c)
    codes = (comprs[0][3:, None] >> np.arange(30, -2, -2, dtype=np.uint32)) & 3
    assert np.any(codes == 3)
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.decompress_2bit(gu.dev(comprs[0]), n, out)
    gu.sync()
    np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit(comprs[0], n))
    for misalign in (False, True):
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.decompress_2bit_sum([gu.dev(c) for c in comprs], n, out)
        gu.sync()
        np.testing.assert_array_equal(gu.host(out), oracle.dequantize_2bit_sum(comprs, n))


@pytest.mark.slow
def test_resnet50_flat_gradient_full_size(gcq):
    """25,557,032 values, W = 8 workers x 5 error-feedback iterations, then
    the dequantize-and-sum -- the benchmark's workload and launch shapes."""
    n, W, T, thr = si.RESNET50_PARAMS, 8, 5, 0.01
    words = gcq.gc_compressed_2bit_words(n)
    g_dev = gu.empty(n, torch.float32)
    r_dev = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for _ in range(W)]
    c_dev = [gu.empty(words, torch.int32) for _ in range(W)]
    r_or = [np.zeros(n, np.float32) for _ in range(W)]
    c_or = [None] * W
    for t in range(T):
        for w in range(W):
            announce(f"2-bit full size n={n} iter={t} worker={w}")
            g = si.normal_f32(si.grad_seed(w, t), n, 0.01)
            g_dev.copy_(torch.from_numpy(g))
            c_dev[w].fill_(-1)
            gcq.compress_2bit(g_dev, r_dev[w], -thr, thr, c_dev[w])
            c_or[w] = oracle.quantize_2bit(g, r_or[w], -thr, thr)
            gu.sync()
            assert np.array_equal(gu.host(c_dev[w], np.uint32), c_or[w]), (t, w)
            assert np.array_equal(gu.host(r_dev[w]).view(np.uint32), r_or[w].view(np.uint32)), (t, w)
    announce("2-bit full size dequantize-sum W=8")
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.decompress_2bit_sum(c_dev, n, out)
    gu.sync()
    got = gu.host(out)
    expect = oracle.dequantize_2bit_sum(c_or, n)
    assert np.all(np.abs(got - expect) <= 1e-6 * np.abs(expect))
    assert np.array_equal(got, expect)


def _multi_case(gcq, sizes, iters, sigma, thr, misalign_every=0, seed0=0):
    T = len(sizes)
    grads_dev, res_dev = [], []
    for t, n in enumerate(sizes):
        mis = bool(misalign_every) and t % misalign_every == 1
        grads_dev.append(gu.empty(n, torch.float32, misalign=mis))
        r = gu.empty(n, torch.float32, misalign=(mis and t % 3 == 1))
        r.zero_()
        res_dev.append(r)
    plan = gcq.Plan2bitMulti(grads_dev, res_dev)
    offsets = plan.block_offsets()
    assert plan.compressed_words == sum(oracle.compressed_2bit_words(n) for n in sizes)
    compr = gu.empty(plan.compressed_words, torch.int32)
    r_or = [np.zeros(n, np.float32) for n in sizes]
    for it in range(iters):
        announce(f"multi-tensor T={T} iter={it}")
        blocks = []
        for t, n in enumerate(sizes):
            g = si.normal_f32(seed0 + 7919 * t + it, n, sigma)
            grads_dev[t].copy_(torch.from_numpy(g))
            blocks.append(oracle.quantize_2bit(g, r_or[t], -thr, thr))
        compr.fill_(-1)
        plan.compress(-thr, thr, compr)
        gu.sync()
        got = gu.host(compr, np.uint32)
        for t, n in enumerate(sizes):
            blk = got[offsets[t]:offsets[t] + oracle.compressed_2bit_words(n)]
            assert np.array_equal(blk, blocks[t]), (it, t, n)
            assert np.array_equal(gu.host(res_dev[t]).view(np.uint32), r_or[t].view(np.uint32)), (it, t)
    plan.destroy()


def test_multi_tensor_ragged(gcq):
    sizes = [0, 1, 5, 16, 17, 4095, 4096, 4097, 8192 + 3, 100_000, 0, 3]
    sizes += si.random_sizes(11, 20, 50_000)
    _multi_case(gcq, sizes, 2, 0.5, 0.5, misalign_every=4)


@pytest.mark.slow
def test_multi_tensor_bert_base_full_size(gcq):
    sizes = si.bert_base_sizes()
    assert len(sizes) == 198 and sum(sizes) == si.BERT_BASE_PARAMS
    _multi_case(gcq, sizes, 3, 0.005, 0.005)


def test_striding_paths_with_capped_grid(gcq):
    """Every kernel family with its grid capped at 3 workgroups (so each one
    strides over many tiles), in a child process; see grid_cap_check.py."""
    import os
    import subprocess
    import sys
    announce("capped-grid parity (child process, GCQ_MAX_GRID_BLOCKS=3)")
    env = dict(os.environ, GCQ_MAX_GRID_BLOCKS="3")
    script = os.path.join(os.path.dirname(__file__), "grid_cap_check.py")
    res = subprocess.run([sys.executable, "-u", script], env=env, capture_output=True,
                         text=True, timeout=110)
    print(res.stdout[-2000:], res.stderr[-2000:])
    assert res.returncode == 0 and res.stdout.strip().endswith("OK")
