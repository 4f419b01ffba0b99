"""GPU parity of the one-call GlobalRandK-MN step (grandk_mn_step) against
the oracle: the shared indices, the norm and the int32 level sums bit for
bit, and the dense dequantized output within 1e-6 relative error
(bit-exact in fact).

Workloads: the ResNet-50 size (25,557,032 values ~ N(0, 0.01^2), K = 10000,
W = 8, s = 7) in the launch configuration the benchmark times; small and
ragged sizes with K from 0 to n, both draw kernels (K at and above 16384),
worker counts from 1 to 64 (compile-time and run-time W), misaligned dense
outputs, zero gradients; and the step captured in a HIP graph, replayed
several times with eager work in between.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def run_step(gcq, grads, K, s, seed, misalign=False, with_sums=True):
    W, n = len(grads), grads[0].size
    g_dev = [gu.dev(g) for g in grads]
    idx = gu.empty(max(K, 1), torch.int32, fill=-1)
    sums = gu.empty(max(K, 1), torch.int32, fill=-7) if with_sums else None
    dense = gu.empty(n, torch.float32, misalign=misalign, fill=float("nan"))
    norm = torch.full((1,), float("nan"), dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_mn_step(g_dev, K, seed, s, idx, dense, ws, sums=sums, norm=norm)
    gu.sync()
    return (gu.host(idx, np.uint32)[:K], None if sums is None else gu.host(sums)[:K],
            gu.host(dense), np.float32(gu.host(norm)[0]))


def oracle_step(grads, K, s, seed):
    n = grads[0].size
    idx = oracle.randk_indices(n, K, seed)
    gk = [oracle.gather(g, idx) for g in grads]
    norm = oracle.maxnorm(gk) if K > 0 else np.float32(0.0)
    S = oracle.level_sum([oracle.qsgd_quantize(g, norm, s, seed, w) for w, g in enumerate(gk)])
    dense = oracle.scatter_dense(oracle.qsgd_dequantize(S, norm, s), idx, n)
    return idx, S, dense, norm


def check(got, expect):
    idx, S, dense, norm = got
    idx_or, S_or, dense_or, norm_or = expect
    np.testing.assert_array_equal(idx, idx_or)
    assert norm.view(np.uint32) == np.float32(norm_or).view(np.uint32)
    if S is not None:
        np.testing.assert_array_equal(S, S_or)
    assert np.all(np.abs(dense.astype(np.float64) - dense_or) <= 1e-6 * np.abs(dense_or.astype(np.float64)))
    np.testing.assert_array_equal(dense, dense_or)


@pytest.mark.parametrize("n,K,W,s", [(1, 1, 1, 127), (1, 0, 2, 7), (7, 7, 3, 7), (1000, 999, 8, 7),
                                     (100_003, 10_000, 8, 7), (65_536, 16_384, 4, 15),
                                     (70_001, 16_385, 5, 7), (300_007, 40_000, 9, 127),
                                     (20_000, 5_003, 64, 3), (5_000, 4_001, 2, 1),
                                     # n much larger than K: most of the dense fill runs
                                     # beside the draw, gathers and scatter
                                     (2_000_003, 100, 8, 7), (10_001, 0, 3, 7), (5_000, 1, 2, 7),
                                     (4_000_000, 2_000, 4, 127)])
def test_grandk_mn_step_small(gcq, n, K, W, s):
    announce(f"grandk_mn_step n={n} K={K} W={W} s={s}")
    seed = 0x9A9A + n + K
    grads = [si.normal_f32(si.grad_seed(w, 6), n, 0.01) for w in range(W)]
    check(run_step(gcq, grads, K, s, seed), oracle_step(grads, K, s, seed))


@pytest.mark.parametrize("misalign", [False, True])
@pytest.mark.parametrize("n,K", [(123_457, 3_001), (1_000_001, 50)])
def test_grandk_mn_step_misaligned_dense_without_sums(gcq, misalign, n, K):
    announce(f"grandk_mn_step dense misalign={misalign}, no sums, n={n} K={K}")
    W, s, seed = 8, 7, 11
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 8), n, 0.02) for w in range(W)]
    idx, S, dense, norm = run_step(gcq, grads, K, s, seed, misalign=misalign, with_sums=False)
    assert S is None
    check((idx, None, dense, norm), oracle_step(grads, K, s, seed))


@pytest.mark.parametrize("off", [1, 2, 3])
@pytest.mark.parametrize("n,K", [(7, 7), (13, 13), (4_099, 4_099), (16_387, 16_384),
                                 (100_003, 5_000), (2_000_005, 3_000)])
def test_grandk_mn_step_dense_head_and_tail(gcq, off, n, K):
    """dense as a view `off` floats into its buffer (so 4 - off values before
    its first 16-byte boundary) with n % 4 values after its last whole float4,
    every position drawn in the small cases: the fill's head, tail, regions
    and drawn-position bitmap against the oracle, and nothing written
    outside the view."""
    announce(f"grandk_mn_step dense view at +{off}, n={n} K={K}")
    W, s, seed = 3, 7, 0x51DE + n + off
    grads = [si.normal_f32(si.grad_seed(w, 9), n, 0.01) for w in range(W)]
    g_dev = [gu.dev(g) for g in grads]
    buf = torch.full((n + 8,), 7.0, dtype=torch.float32, device=gu.DEV)
    dense = buf[off:off + n]
    idx = gu.empty(K, torch.int32, fill=-1)
    sums = gu.empty(K, torch.int32, fill=-7)
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_mn_step(g_dev, K, seed, s, idx, dense, ws, sums=sums, norm=norm)
    gu.sync()
    check((gu.host(idx, np.uint32), gu.host(sums), gu.host(dense), np.float32(gu.host(norm)[0])),
          oracle_step(grads, K, s, seed))
    hb = gu.host(buf)
    assert np.all(hb[:off] == 7.0) and np.all(hb[off + n:] == 7.0)


def test_grandk_mn_step_workspace_reused_across_sizes(gcq):
    """One workspace, sized for the largest call, serves calls of other sizes
    in turn: whatever a call leaves in it (fill progress, flags, marks of
    drawn positions) must not reach the next."""
    W, s = 4, 7
    cases = [(1_000_003, 10_000, 1), (5_001, 4_000, 2), (1_000_003, 9_000, 3), (60_000, 16_384, 4)]
    ws = torch.empty(max(gcq.grandk_mn_step_ws_bytes(W, n, K) for n, K, _ in cases),
                     dtype=torch.uint8, device=gu.DEV)
    for n, K, seed in cases:
        announce(f"grandk_mn_step reused workspace n={n} K={K}")
        grads = [si.normal_f32(si.grad_seed(w, 10 + seed), n, 0.01) for w in range(W)]
        g_dev = [gu.dev(g) for g in grads]
        idx = gu.empty(K, torch.int32, fill=-1)
        sums = gu.empty(K, torch.int32, fill=-7)
        dense = gu.empty(n, torch.float32, fill=float("nan"))
        norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
        gcq.grandk_mn_step(g_dev, K, seed, s, idx, dense, ws, sums=sums, norm=norm)
        gu.sync()
        check((gu.host(idx, np.uint32), gu.host(sums), gu.host(dense),
               np.float32(gu.host(norm)[0])), oracle_step(grads, K, s, seed))


def test_grandk_mn_step_zero_gradients(gcq):
    announce("grandk_mn_step all-zero gradients")
    grads = [np.zeros(50_000, np.float32), np.array([-0.0] * 50_000, np.float32)]
    idx, S, dense, norm = run_step(gcq, grads, 1000, 7, 3)
    np.testing.assert_array_equal(idx, oracle.randk_indices(50_000, 1000, 3))
    assert norm == 0.0 and np.all(S == 0) and np.all(dense == 0)


@pytest.mark.slow
def test_grandk_mn_step_resnet50(gcq):
    """n = 25,557,032, K = 10000, W = 8, s = 7, seed 0: the benchmark's
    workload, checked in full (every dense element)."""
    n, K, W, s, seed = si.RESNET50_PARAMS, 10_000, 8, 7, 0
    announce(f"grandk_mn_step full size n={n} K={K} W={W}")
    grads = [si.normal_f32(si.grad_seed(w, 0), n, 0.01) for w in range(W)]
    check(run_step(gcq, grads, K, s, seed), oracle_step(grads, K, s, seed))


def test_grandk_mn_step_in_hip_graph(gcq):
    """Captured once, replayed four times with eager work and
    synchronisation between the replays; every replay equals the eager
    result bit for bit."""
    n, K, W, s, seed = 300_007, 2_000, 8, 7, 5
    announce("grandk_mn_step captured in a HIP graph")
    g_dev = [gu.dev(si.normal_f32(si.grad_seed(w, 2), n, 0.01)) for w in range(W)]
    idx = gu.empty(K, torch.int32)
    sums = gu.empty(K, torch.int32)
    dense = gu.empty(n, torch.float32)
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)

    def step():
        gcq.grandk_mn_step(g_dev, K, seed, s, idx, dense, ws, sums=sums, norm=norm)

    step()
    gu.sync()
    eager = (gu.host(idx).copy(), gu.host(sums).copy(), gu.host(dense).copy(), gu.host(norm).copy())
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
        norm.fill_(float("nan"))
        gu.sync()
        graph.replay()
        gu.sync()
        got = (gu.host(idx), gu.host(sums), gu.host(dense), gu.host(norm))
        for a, b in zip(got, eager):
            np.testing.assert_array_equal(a, b, err_msg=f"replay {rep}")
        step()
        gu.sync()
