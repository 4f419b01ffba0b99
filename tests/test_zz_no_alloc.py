"""qsgd_global_maxnorm_noalloc, through the C ABI: the max-norm with its
partial maxima in the library's fixed device array instead of a caller
workspace. Each call must give exactly what qsgd_global_maxnorm gives on the
same input, and what the oracle gives, also when the array still holds the
larger partials of the call before it.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def with_workspace(gcq, g_dev):
    norm = torch.full((1,), float("nan"), dtype=torch.float32, device=gu.DEV)
    n = g_dev[0].numel()
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(len(g_dev), n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    return norm


def no_alloc(gcq, g_dev):
    norm = torch.full((1,), float("nan"), dtype=torch.float32, device=gu.DEV)
    gcq.qsgd_global_maxnorm_noalloc(g_dev, norm)
    return norm


def bits(t):
    return gu.host(t).view(np.uint32)[0]


def test_two_calls_in_a_row_second_smaller(gcq):
    """A large call (8 workers x 3,000,017 values, with one value of 1e30 so
    that its partials dominate), then a smaller one (3 x 5001): the second
    reads only its own partials, none left by the first."""
    big = [si.heavy_tailed_f32(si.grad_seed(w, 21), 3_000_017, 0.02) for w in range(8)]
    big[5][1_234_567] = np.float32(-1e30)
    small = [si.normal_f32(si.grad_seed(w, 22), 5001, 0.5) for w in range(3)]
    for case, grads in (("8 x 3,000,017", big), ("3 x 5001", small)):
        announce(f"qsgd_global_maxnorm_noalloc {case}")
        g_dev = [gu.dev(g) for g in grads]
        a = no_alloc(gcq, g_dev)
        b = with_workspace(gcq, g_dev)
        gu.sync()
        assert bits(a) == bits(b), case
        assert bits(a) == oracle.maxnorm(grads).view(np.uint32), case
    assert gu.host(a)[0] < 1e29


def test_misaligned_and_ragged(gcq):
    """Buffers 4 bytes off 16-byte alignment and sizes around a tile."""
    for W, n in ((1, 1), (2, 7), (5, 1023), (64, 4097), (3, 65_539)):
        announce(f"qsgd_global_maxnorm_noalloc W={W} n={n} misaligned")
        grads = [si.heavy_tailed_f32(si.grad_seed(w, 23), n, 0.02) for w in range(W)]
        g_dev = [gu.dev(g, True) for g in grads]
        a = no_alloc(gcq, g_dev)
        b = with_workspace(gcq, g_dev)
        gu.sync()
        assert bits(a) == bits(b) == oracle.maxnorm(grads).view(np.uint32)


def test_every_partial_of_the_array(gcq):
    """64 workers, each large enough for the most workgroups per worker: the
    call uses all of the fixed array (the 64 pointers share one buffer)."""
    n = 4096 * 2048 * 4 + 3  # 4096 workgroups of 2048 float4 slots per worker
    announce(f"qsgd_global_maxnorm_noalloc W=64 n={n} (one shared buffer)")
    g = torch.empty(n, dtype=torch.float32, device=gu.DEV).uniform_(-1.0, 1.0)
    g[n // 3] = 7.5
    g_dev = [g] * 64
    ws_bytes = gcq.qsgd_maxnorm_ws_bytes(64, n)
    assert ws_bytes == 64 * 4096 * 4  # the array's full size
    a = no_alloc(gcq, g_dev)
    b = with_workspace(gcq, g_dev)
    gu.sync()
    assert bits(a) == bits(b)
    assert gu.host(a)[0] == np.float32(7.5)


def test_arguments_are_checked(gcq):
    L = gcq.load()
    arr = (ctypes.c_void_p * 1)(None)
    assert L.qsgd_global_maxnorm_noalloc(arr, 0, 10, None, None) == gcq.GC_EINVAL
    assert L.qsgd_global_maxnorm_noalloc(arr, 65, 10, None, None) == gcq.GC_EINVAL
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    assert L.qsgd_global_maxnorm_noalloc(arr, 1, 10, ctypes.c_void_p(norm.data_ptr()),
                                         None) == gcq.GC_EINVAL
    assert "NULL" in gcq.last_error()
