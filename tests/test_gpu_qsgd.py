"""GPU parity of the QSGD max-norm path and GlobalRandK against the oracle.

Bit-exact: the global max-norm, the int8 levels, the int32 level sums, the
rand-K indices and the gathered values. Dequantized fp32 values: within 1e-6
relative error (in fact bit-exact: the same two fp32 roundings).

Workloads: ragged sizes and worker counts; the VGG16-sized heavy-tailed
gradient (W = 8 workers x 138,357,544 values ~ N(0, 0.02^2), each entry
scaled by 50 with probability 0.001, s = 127) in the launch configuration the
benchmark times, every element against the oracle; and GlobalRandK at the ResNet-50 size (25,557,032 values ~
N(0, 0.01^2), K = 10000, W = 8, s = 7), checked in full.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def run_qsgd(gcq, grads, s, seed, misalign=False, scatter_idx=None, dense_n=0):
    """Full QSGD-MN step on the device: norm -> levels per worker -> sums ->
    dequantized output. Returns host copies."""
    W, n = len(grads), grads[0].size
    g_dev = [gu.dev(g, misalign) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    levels = [gu.empty(n, torch.int8, misalign=misalign, fill=99) for _ in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, levels[w])
    sums = gu.empty(n, torch.int32, misalign=misalign, fill=-7)
    if scatter_idx is None:
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)
    else:
        out = gu.empty(dense_n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums, scatter_idx=scatter_idx,
                             dense_n=dense_n)
    gu.sync()
    return (np.float32(gu.host(norm)[0]), [gu.host(q) for q in levels], gu.host(sums),
            gu.host(out))


def check_deq(got, expect):
    assert np.all(np.abs(got.astype(np.float64) - expect) <= 1e-6 * np.abs(expect.astype(np.float64)))
    np.testing.assert_array_equal(got, expect)


@pytest.mark.parametrize("byte_off", [1, 2, 3])
def test_levels_at_odd_byte_offsets(gcq, byte_off):
    """int8 levels 1-3 bytes off 4-byte alignment (the word paths that
    realign them in registers); gradients at a 4-byte offset, outputs
    aligned."""
    n, W, s, seed = 70_001, 3, 127, 19
    announce(f"qsgd levels at byte offset {byte_off}")
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 13), n, 0.02) for w in range(W)]
    g_dev = [gu.dev(g, True) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    bufs = [torch.full((n + 4,), 99, dtype=torch.int8, device=gu.DEV) for _ in range(W)]
    levels = [b[byte_off:byte_off + n] for b in bufs]
    assert all(lv.data_ptr() % 4 == byte_off % 4 for lv in levels)
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, levels[w])
    sums = gu.empty(n, torch.int32, fill=-7)
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)
    gu.sync()
    norm_or = oracle.maxnorm(grads)
    assert np.float32(gu.host(norm)[0]) == norm_or
    lv_or = [oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(grads)]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w])
        # nothing written outside the view
        np.testing.assert_array_equal(gu.host(bufs[w][:byte_off]), np.full(byte_off, 99, np.int8))
        np.testing.assert_array_equal(gu.host(bufs[w][byte_off + n:]), np.full(4 - byte_off, 99, np.int8))
    S = oracle.level_sum(lv_or)
    np.testing.assert_array_equal(gu.host(sums), S)
    check_deq(gu.host(out), oracle.qsgd_dequantize(S, norm_or, s))


@pytest.mark.parametrize("gmis", [False, True])
@pytest.mark.parametrize("W,n", [(8, 70_001), (5, 300_007), (8, 1024 * 256 * 3 + 257),
                                 (2, 1031), (13, 9_999)])
def test_levels_at_mixed_byte_offsets(gcq, W, n, gmis):
    """Each worker's int8 levels at its own offset 0-3 past a 4-byte boundary
    (the word paths that realign levels in registers; W = 8 known at compile
    time, other W read at run time), gradients aligned or 4 bytes off, sizes
    over several tiles with a ragged tail: levels, sums and values against
    the oracle, and no byte written outside any view."""
    seed = 0xB17E5 + n + W
    announce(f"qsgd levels at mixed byte offsets W={W} n={n} gmis={gmis}")
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 14), n, 0.02) for w in range(W)]
    g_dev = [gu.dev(g, gmis) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    offs = [(3 * w + 1) % 4 for w in range(W)]
    bufs = [torch.full((n + 8,), 99, dtype=torch.int8, device=gu.DEV) for _ in range(W)]
    levels = [bufs[w][offs[w]:offs[w] + n] for w in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, 127, seed, w, levels[w])
    sums = gu.empty(n, torch.int32, fill=-7)
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.qsgd_dequant_sum(levels, norm, 127, out, sums=sums)
    gu.sync()
    norm_or = oracle.maxnorm(grads)
    assert np.float32(gu.host(norm)[0]) == norm_or
    lv_or = [oracle.qsgd_quantize(g, norm_or, 127, seed, w) for w, g in enumerate(grads)]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w], err_msg=f"worker {w}")
        hb = gu.host(bufs[w])
        assert np.all(hb[:offs[w]] == 99) and np.all(hb[offs[w] + n:] == 99), f"worker {w}"
    S = oracle.level_sum(lv_or)
    np.testing.assert_array_equal(gu.host(sums), S)
    check_deq(gu.host(out), oracle.qsgd_dequantize(S, norm_or, 127))
    # the level sum alone on arbitrary int8 bytes at those offsets, the
    # outputs 4 bytes off 16-byte alignment (staged stores)
    rng = np.random.default_rng(n + W)
    anyq = [rng.integers(-128, 128, n, dtype=np.int64).astype(np.int8) for _ in range(W)]
    for w in range(W):
        levels[w].copy_(torch.from_numpy(anyq[w]))
    sums_m = gu.empty(n, torch.int32, misalign=True, fill=-7)
    out_m = gu.empty(n, torch.float32, misalign=True, fill=float("nan"))
    gcq.qsgd_dequant_sum(levels, norm, 127, out_m, sums=sums_m)
    gu.sync()
    S_any = oracle.level_sum(anyq)
    np.testing.assert_array_equal(gu.host(sums_m), S_any)
    check_deq(gu.host(out_m), oracle.qsgd_dequantize(S_any, norm_or, 127))


@pytest.mark.slow
def test_levels_at_byte_offsets_vgg16_full_size(gcq):
    """The VGG16-sized step with worker w's levels at byte offset 1 + w % 3:
    every level, sum and value against the oracle's run over all elements."""
    import vgg16_case as vc
    announce("qsgd full size, levels at byte offsets: generating inputs")
    grads = vc.grads()
    g_dev = [gu.dev(g) for g in grads]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(vc.W, vc.N), dtype=torch.uint8, device=gu.DEV)
    announce("qsgd full size, levels at byte offsets: device step")
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    bufs = [torch.empty(vc.N + 4, dtype=torch.int8, device=gu.DEV) for _ in range(vc.W)]
    levels = [bufs[w][1 + w % 3:1 + w % 3 + vc.N] for w in range(vc.W)]
    for w in range(vc.W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, vc.S, vc.SEED, w, levels[w])
    del g_dev
    sums = gu.empty(vc.N, torch.int32, fill=-7)
    out = gu.empty(vc.N, torch.float32, fill=float("nan"))
    gcq.qsgd_dequant_sum(levels, norm, vc.S, out, sums=sums)
    gu.sync()
    announce("qsgd full size, levels at byte offsets: oracle over every element")
    norm_or, lv_or, s_or, d_or = vc.oracle_step()
    assert np.float32(gu.host(norm)[0]) == norm_or
    for w in range(vc.W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w], err_msg=f"worker {w}")
    np.testing.assert_array_equal(gu.host(sums), s_or)
    check_deq(gu.host(out), d_or)
    del bufs, levels, sums, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("W,n,s", [(1, 1, 127), (2, 5, 7), (3, 4097, 127), (8, 1000, 1),
                                   (5, 65536 + 3, 15), (64, 777, 127), (8, 1 << 20, 127),
                                   (4, 5003, 7)])
def test_qsgd_step_small(gcq, W, n, s, misalign):
    announce(f"qsgd W={W} n={n} s={s} misalign={misalign}")
    seed = 0xABCDEF0123 + n
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 1), n, 0.02) for w in range(W)]
    norm, levels, sums, out = run_qsgd(gcq, grads, s, seed, misalign)
    norm_or = oracle.maxnorm(grads)
    assert norm.view(np.uint32) == norm_or.view(np.uint32)
    lv_or = [oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(grads)]
    for w in range(W):
        np.testing.assert_array_equal(levels[w], lv_or[w], err_msg=f"worker {w}")
    s_or = oracle.level_sum(lv_or)
    np.testing.assert_array_equal(sums, s_or)
    check_deq(out, oracle.qsgd_dequantize(s_or, norm_or, s))


@pytest.mark.parametrize("W,n", [(1, 1000), (3, 4097), (8, 100_003), (13, 777), (17, 100_003),
                                 (33, 65_537), (64, 20_011)])
def test_level_sum_of_arbitrary_levels(gcq, W, n):
    """The level sum and dequantize take any int8 levels, -128 and 127
    included: the int32 sums are exact whatever the inputs."""
    announce(f"qsgd level sum of arbitrary int8 levels W={W} n={n}")
    rng = np.random.default_rng(977 * n + W)
    levels = [rng.integers(-128, 128, n, dtype=np.int64).astype(np.int8) for _ in range(W)]
    levels[0][:2] = (-128, 127)
    norm_v, s = np.float32(0.0371), 127
    norm = torch.tensor([norm_v], dtype=torch.float32, device=gu.DEV)
    S_or = oracle.level_sum(levels)
    for misalign in (False, True):
        sums = gu.empty(n, torch.int32, misalign=misalign, fill=-7)
        out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
        gcq.qsgd_dequant_sum([gu.dev(q, misalign) for q in levels], norm, s, out, sums=sums)
        gu.sync()
        np.testing.assert_array_equal(gu.host(sums), S_or)
        check_deq(gu.host(out), oracle.qsgd_dequantize(S_or, norm_v, s))


def test_qsgd_zero_gradient(gcq):
    announce("qsgd all-zero gradients")
    grads = [np.zeros(1000, np.float32), np.array([-0.0] * 1000, np.float32)]
    norm, levels, sums, out = run_qsgd(gcq, grads, 127, 5)
    assert norm == 0.0
    assert all(np.all(q == 0) for q in levels)
    assert np.all(sums == 0) and np.all(out == 0)


def test_qsgd_norm_element_is_s(gcq):
    announce("qsgd |g| = norm -> s")
    g = si.normal_f32(4, 4099, 1.0)
    j = int(np.argmax(np.abs(g)))
    for seed in range(5):
        norm, levels, _, _ = run_qsgd(gcq, [g], 127, seed)
        assert abs(int(levels[0][j])) == 127


@pytest.mark.slow
def test_qsgd_vgg16_full_size(gcq):
    """8 workers x 138,357,544 heavy-tailed values, s = 127, seed 0, in the
    launch configuration the benchmark times: the max-norm, every worker's
    every level, every int32 sum and every dequantized value against the
    oracle's run over all elements; then the same step on buffers 4 bytes
    off 16-byte alignment (the staged kernels at full size), against the
    oracle again."""
    import vgg16_case as vc
    announce(f"qsgd full size: generating {vc.W} workers x {vc.N} values")
    grads = vc.grads()
    for misalign in (False, True):
        announce(f"qsgd full size: device step (misalign={misalign})")
        norm, levels, sums, out = run_qsgd(gcq, list(grads), vc.S, vc.SEED, misalign=misalign)
        torch.cuda.empty_cache()
        announce("qsgd full size: oracle over every element")
        norm_or, lv_or, s_or, d_or = vc.oracle_step()
        assert norm.view(np.uint32) == norm_or.view(np.uint32)
        for w in range(vc.W):
            np.testing.assert_array_equal(levels[w], lv_or[w],
                                          err_msg=f"worker {w} misalign={misalign}")
        del levels
        np.testing.assert_array_equal(sums, s_or)
        check_deq(out, d_or)
        del sums, out


@pytest.mark.parametrize("n,K", [(1, 1), (1, 0), (7, 7), (1000, 1000), (100_000, 10_000),
                                 (1 << 20, 1), (3, 2), (16384, 16384), (40_000, 16_385),
                                 (1 << 20, 20_000), (1 << 20, 100_000)])
def test_grandk_indices(gcq, n, K):
    for seed in (0, 1, 0xDEADBEEFCAFE):
        announce(f"grandk_indices n={n} K={K} seed={seed}")
        idx = gu.empty(max(K, 1), torch.int32, fill=-1)
        ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=gu.DEV)
        gcq.grandk_indices(n, K, seed, idx[:K], ws)
        gu.sync()
        np.testing.assert_array_equal(gu.host(idx, np.uint32)[:K], oracle.randk_indices(n, K, seed))


def test_grandk_indices_collisions(gcq):
    """Small n with K close to n forces chains of earlier swaps."""
    for n, K in [(50, 49), (64, 64), (300, 250), (5000, 4000)]:
        for seed in range(20):
            announce(f"grandk_indices n={n} K={K} seed={seed}")
            idx = gu.empty(K, torch.int32)
            ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=gu.DEV)
            gcq.grandk_indices(n, K, seed, idx, ws)
            gu.sync()
            np.testing.assert_array_equal(gu.host(idx, np.uint32), oracle.randk_indices(n, K, seed))


def test_gather(gcq):
    announce("gather_f32")
    x = si.normal_f32(3, 100_001, 1.0)
    idx = oracle.randk_indices(x.size, 5000, 8)
    for misalign in (False, True):
        out = gu.empty(5000, torch.float32, misalign=misalign)
        gcq.gather_f32(gu.dev(x, misalign), gu.dev(idx), out)
        gu.sync()
        np.testing.assert_array_equal(gu.host(out), oracle.gather(x, idx))


@pytest.mark.parametrize("full", [False, pytest.param(True, marks=pytest.mark.slow)])
def test_grandk_step(gcq, full):
    """GRandK-MN: shared K indices -> gather per worker -> QSGD-MN at s = 7 ->
    level sum -> scatter-dequantize into a dense buffer."""
    n = si.RESNET50_PARAMS if full else 200_003
    K, W, s, seed = 10_000, 8, 7, 0
    announce(f"grandk step n={n} K={K} W={W}")
    grads = [si.normal_f32(si.grad_seed(w, 0), n, 0.01) for w in range(W)]
    g_dev = [gu.dev(g) for g in grads]
    idx = gu.empty(K, torch.int32)
    ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_indices(n, K, seed, idx, ws)
    gathered = [gu.empty(K, torch.float32) for _ in range(W)]
    for w in range(W):
        gcq.gather_f32(g_dev[w], idx, gathered[w])
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    mws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, K), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(gathered, norm, mws)
    levels = [gu.empty(K, torch.int8) for _ in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(gathered[w], norm, s, seed, w, levels[w])
    sums = gu.empty(K, torch.int32)
    dense = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.qsgd_dequant_sum(levels, norm, s, dense, sums=sums, scatter_idx=idx, dense_n=n)
    gu.sync()

    idx_or = oracle.randk_indices(n, K, seed)
    np.testing.assert_array_equal(gu.host(idx, np.uint32), idx_or)
    gk_or = [oracle.gather(g, idx_or) for g in grads]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(gathered[w]), gk_or[w])
    norm_or = oracle.maxnorm(gk_or)
    assert np.float32(gu.host(norm)[0]).view(np.uint32) == norm_or.view(np.uint32)
    lv_or = [oracle.qsgd_quantize(gk_or[w], norm_or, s, seed, w) for w in range(W)]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w])
    s_or = oracle.level_sum(lv_or)
    np.testing.assert_array_equal(gu.host(sums), s_or)
    dense_or = oracle.scatter_dense(oracle.qsgd_dequantize(s_or, norm_or, s), idx_or, n)
    check_deq(gu.host(dense), dense_or)


@pytest.mark.parametrize("s", [1, 4, 7, 127])
def test_qsgd_level_edges(gcq, s):
    """Values whose scaled magnitude x is integral, one ulp either side of an
    integer, tiny or subnormal, over many rounding seeds: the level must be
    floor(x + u) exactly, as the oracle computes it."""
    announce(f"qsgd level edges s={s}")
    base = [1.0, -1.0, 0.0, -0.0, 1e-45, -1e-40, 1e-30, 2.0 ** -31, 0.5, 0.25, 1.0 / 3.0]
    for j in range(0, s + 1):
        v = np.float32(j / s)
        base += [float(v), float(np.nextafter(v, np.float32(2))), float(np.nextafter(v, np.float32(0)))]
    g = np.array(base * 4, np.float32)
    g[len(base):2 * len(base)] *= -1
    g = np.clip(g, -1.0, 1.0).astype(np.float32)  # norm = 1 exactly
    g_dev = gu.dev(g)
    norm = torch.ones(1, dtype=torch.float32, device=gu.DEV)
    lv = gu.empty(g.size, torch.int8)
    for seed in range(64):
        gcq.qsgd_maxnorm_quantize(g_dev, norm, s, seed, seed % 5, lv)
        gu.sync()
        np.testing.assert_array_equal(gu.host(lv), oracle.qsgd_quantize(g, 1.0, s, seed, seed % 5),
                                      err_msg=f"seed {seed}")


@pytest.mark.parametrize("norm_scale", [1e-38, 2.0 ** -121, 1e-30, 2.0 ** -98, 2.0 ** -96, 1e30])
def test_qsgd_extreme_norms(gcq, norm_scale):
    """Tiny norms (where 1/norm would overflow, so every value takes the
    exact division) and huge ones, through the whole QSGD step."""
    announce(f"qsgd extreme norm scale {norm_scale}")
    g = (si.normal_f32(77, 10_007, 1.0) * np.float32(norm_scale)).astype(np.float32)
    g[5] = np.float32(-3.0 * norm_scale)
    norm, levels, sums, out = run_qsgd(gcq, [g], 127, 3)
    norm_or = oracle.maxnorm([g])
    assert norm.view(np.uint32) == norm_or.view(np.uint32)
    np.testing.assert_array_equal(levels[0], oracle.qsgd_quantize(g, norm_or, 127, 3, 0))


@pytest.mark.parametrize("norm_bits", ["2^-96", "below 2^-96", "2^-95", "2^-120"])
def test_qsgd_fast_path_threshold(gcq, norm_bits):
    """Norms at and around the smallest one that takes the multiply-by-
    reciprocal fast path (2^-96; one ulp below it every value divides):
    per-worker quantize and the fused quantize-sum both equal the oracle."""
    announce(f"qsgd fast-path threshold norm={norm_bits}")
    base = {"2^-96": np.float32(2.0 ** -96), "2^-95": np.float32(2.0 ** -95),
            "below 2^-96": np.nextafter(np.float32(2.0 ** -96), np.float32(0)),
            "2^-120": np.float32(2.0 ** -120)}[norm_bits]
    grads = []
    for w in range(3):
        g = si.normal_f32(300 + w, 20_011, 1.0)
        g = (g / np.float32(np.abs(g).max() * 1.01) * base).astype(np.float32)
        grads.append(g)
    grads[1][7] = -base
    for s in (7, 127):
        norm, levels, sums, out = run_qsgd(gcq, grads, s, 19)
        assert norm.view(np.uint32) == base.view(np.uint32)
        lv_or = [oracle.qsgd_quantize(g, base, s, 19, w) for w, g in enumerate(grads)]
        for w in range(3):
            np.testing.assert_array_equal(levels[w], lv_or[w], err_msg=f"s={s} worker {w}")
        s_or = oracle.level_sum(lv_or)
        np.testing.assert_array_equal(sums, s_or)
        check_deq(out, oracle.qsgd_dequantize(s_or, base, s))
        fsums = gu.empty(20_011, torch.int32)
        fout = gu.empty(20_011, torch.float32)
        nt = torch.tensor([base], dtype=torch.float32, device=gu.DEV)
        gcq.qsgd_quantize_sum([gu.dev(g) for g in grads], nt, s, 19, fout, sums=fsums)
        gu.sync()
        np.testing.assert_array_equal(gu.host(fsums), s_or)
        check_deq(gu.host(fout), oracle.qsgd_dequantize(s_or, base, s))


def test_grandk_step_in_hip_graph(gcq):
    """The whole GRandK-MN step captured once as a HIP graph and replayed
    several times, with eager work and synchronisation between replays:
    every replay must reproduce the eager result bit for bit."""
    n, K, W, s, seed = 300_007, 2_000, 4, 7, 5
    announce("grandk step captured in a HIP graph")
    grads = [gu.dev(si.normal_f32(si.grad_seed(w, 2), n, 0.01)) for w in range(W)]
    idx = gu.empty(K, torch.int32)
    ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=gu.DEV)
    gathered = [gu.empty(K, torch.float32) for _ in range(W)]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    mws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, K), dtype=torch.uint8, device=gu.DEV)
    levels = [gu.empty(K, torch.int8) for _ in range(W)]
    sums = gu.empty(K, torch.int32)
    dense = gu.empty(n, torch.float32)

    def step():
        gcq.grandk_indices(n, K, seed, idx, ws)
        for w in range(W):
            gcq.gather_f32(grads[w], idx, gathered[w])
        gcq.qsgd_global_maxnorm(gathered, norm, mws)
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(gathered[w], norm, s, seed, w, levels[w])
        gcq.qsgd_dequant_sum(levels, norm, s, dense, sums=sums, scatter_idx=idx, dense_n=n)

    step()
    gu.sync()
    eager = (gu.host(idx).copy(), gu.host(sums).copy(), gu.host(dense).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    gu.sync()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        dense.fill_(float("nan"))
        sums.fill_(-1)
        idx.fill_(-1)
        gu.sync()
        graph.replay()
        gu.sync()
        got = (gu.host(idx), gu.host(sums), gu.host(dense))
        for a, b in zip(got, eager):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}")
        # eager work in between
        step()
        gu.sync()
