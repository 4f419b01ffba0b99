"""GPU parity of the fused QSGD-MN quantize + level sum (qsgd_quantize_sum)
against the oracle: the int32 sums bit for bit, and the dequantized values
within 1e-6 relative error (bit-exact in fact). The oracle side is the
composition of its per-worker quantize, level sum and dequantize.

Workloads: ragged sizes and worker counts (compile-time and run-time W),
both alignments, with and without the sums output; zero and extreme norms;
level edges; and the VGG16-sized heavy-tailed gradient (W = 8 x 138,357,544
values ~ N(0, 0.02^2), entries scaled by 50 with probability 0.001, s = 127),
every element against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def fused(gcq, g_dev, s, seed, n, misalign=False, with_sums=True, norm=None):
    W = len(g_dev)
    if norm is None:
        norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
        ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
        gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    sums = gu.empty(n, torch.int32, misalign=misalign, fill=-7) if with_sums else None
    out = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    gcq.qsgd_quantize_sum(g_dev, norm, s, seed, out, sums=sums)
    gu.sync()
    return (np.float32(gu.host(norm)[0]), None if sums is None else gu.host(sums), gu.host(out))


def oracle_step(grads, s, seed, norm=None):
    norm_or = oracle.maxnorm(grads) if norm is None else np.float32(norm)
    lv = [oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(grads)]
    S = oracle.level_sum(lv)
    return norm_or, S, oracle.qsgd_dequantize(S, norm_or, s)


def check_deq(got, expect):
    assert np.all(np.abs(got.astype(np.float64) - expect) <= 1e-6 * np.abs(expect.astype(np.float64)))
    np.testing.assert_array_equal(got, expect)


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("W,n,s", [(1, 1, 127), (2, 5, 7), (3, 4097, 127), (4, 4096, 4),
                                   (8, 1000, 1), (8, 1003, 127), (5, 65536 + 3, 15),
                                   (9, 20_001, 127), (64, 777, 127), (8, 1 << 20, 127)])
def test_fused_small(gcq, W, n, s, misalign):
    announce(f"qsgd fused W={W} n={n} s={s} misalign={misalign}")
    seed = 0x5EED0000 + 31 * n + W
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 4), n, 0.02) for w in range(W)]
    g_dev = [gu.dev(g, misalign) for g in grads]
    norm, sums, out = fused(gcq, g_dev, s, seed, n, misalign)
    norm_or, S_or, out_or = oracle_step(grads, s, seed)
    assert norm.view(np.uint32) == norm_or.view(np.uint32)
    np.testing.assert_array_equal(sums, S_or)
    check_deq(out, out_or)
    _, none, out2 = fused(gcq, g_dev, s, seed, n, misalign, with_sums=False)
    assert none is None
    check_deq(out2, out_or)


def test_fused_zero_gradient(gcq):
    announce("qsgd fused all-zero gradients")
    grads = [np.zeros(1000, np.float32), np.array([-0.0] * 1000, np.float32)]
    norm, sums, out = fused(gcq, [gu.dev(g) for g in grads], 127, 5, 1000)
    assert norm == 0.0 and np.all(sums == 0) and np.all(out == 0)


@pytest.mark.parametrize("norm_scale", [1e-38, 2.0 ** -121, 1e-30, 1e30])
def test_fused_extreme_norms(gcq, norm_scale):
    announce(f"qsgd fused extreme norm scale {norm_scale}")
    grads = [(si.normal_f32(77 + w, 10_007, 1.0) * np.float32(norm_scale)).astype(np.float32)
             for w in range(3)]
    grads[1][5] = np.float32(-3.0 * norm_scale)
    norm, sums, out = fused(gcq, [gu.dev(g) for g in grads], 127, 3, 10_007)
    norm_or, S_or, out_or = oracle_step(grads, 127, 3)
    assert norm.view(np.uint32) == norm_or.view(np.uint32)
    np.testing.assert_array_equal(sums, S_or)
    check_deq(out, out_or)


@pytest.mark.parametrize("s", [1, 7, 127])
def test_fused_level_edges(gcq, s):
    """Scaled magnitudes on, just above and just below every integer, tiny and
    subnormal values, norm = 1, two workers holding the same and the negated
    values, many rounding seeds."""
    announce(f"qsgd fused level edges s={s}")
    base = [1.0, -1.0, 0.0, -0.0, 1e-45, -1e-40, 1e-30, 2.0 ** -31, 0.5, 1.0 / 3.0]
    for j in range(0, s + 1):
        v = np.float32(j / s)
        base += [float(v), float(np.nextafter(v, np.float32(2))), float(np.nextafter(v, np.float32(0)))]
    g = np.clip(np.array(base * 4, np.float32), -1.0, 1.0).astype(np.float32)
    grads = [g, (-g).astype(np.float32)]
    g_dev = [gu.dev(x) for x in grads]
    norm = torch.ones(1, dtype=torch.float32, device=gu.DEV)
    for seed in range(64):
        _, sums, out = fused(gcq, g_dev, s, seed, g.size, norm=norm)
        _, S_or, out_or = oracle_step(grads, s, seed, norm=1.0)
        np.testing.assert_array_equal(sums, S_or, err_msg=f"seed {seed}")
        np.testing.assert_array_equal(out, out_or, err_msg=f"seed {seed}")


@pytest.mark.slow
def test_fused_vgg16_full_size(gcq):
    """8 workers x 138,357,544 heavy-tailed values, s = 127, seed 0: the fused
    kernel in the launch configuration the benchmark times, and on buffers 4
    bytes off 16-byte alignment (the staged kernel at full size). Every int32
    sum and every dequantized value against the oracle's run over all
    elements."""
    import vgg16_case as vc
    announce(f"qsgd fused full size: generating {vc.W} workers x {vc.N} values")
    grads = vc.grads()
    for misalign in (False, True):
        announce(f"qsgd fused full size: device step (misalign={misalign})")
        g_dev = [gu.dev(g, misalign) for g in grads]
        norm, sums, out = fused(gcq, g_dev, vc.S, vc.SEED, vc.N, misalign=misalign)
        del g_dev
        torch.cuda.empty_cache()
        announce("qsgd fused full size: oracle over every element")
        norm_or, _, S_or, out_or = vc.oracle_step()
        assert norm.view(np.uint32) == norm_or.view(np.uint32)
        np.testing.assert_array_equal(sums, S_or, err_msg=f"misalign={misalign}")
        check_deq(out, out_or)
        del sums, out
