"""The VGG16-sized QSGD-MN workload and the oracle's step on it, computed once
per test process and shared by the full-size parity tests.

Workload: W = 8 simulated workers x 138,357,544 fp32 values ~ N(0, 0.02^2),
each entry scaled by 50 with probability 0.001 (heavy tails), s = 127,
rounding seed 0. The oracle computes the whole step on every element: the
global max-norm, each worker's int8 levels, the int32 level sums and the
dequantized fp32 values.

The workers' inputs are drawn, and the oracle's per-worker quantize runs, in
one thread per worker: each thread calls the unchanged single-threaded
oracle function on its own worker's array (ctypes releases the GIL during
the call), so the arithmetic is exactly the oracle's; only the wall time
shrinks (the whole step takes about 15 s on one core).
"""
from __future__ import annotations

import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synthetic_inputs as si

N = si.VGG16_PARAMS
W = 8
S = 127
SEED = 0
SIGMA = 0.02


def _threads() -> int:
    return max(1, min(W, os.cpu_count() or 1))


@functools.lru_cache(maxsize=1)
def grads() -> tuple:
    """The W workers' gradients (host float32 arrays)."""
    with ThreadPoolExecutor(_threads()) as ex:
        return tuple(ex.map(lambda w: si.heavy_tailed_f32(si.grad_seed(w, 0), N, SIGMA),
                            range(W)))


@functools.lru_cache(maxsize=1)
def oracle_step():
    """(norm, levels per worker, int32 sums, dequantized fp32) from the oracle
    over every element."""
    g = grads()
    norm = oracle.maxnorm(list(g))
    with ThreadPoolExecutor(_threads()) as ex:
        levels = tuple(ex.map(lambda w: oracle.qsgd_quantize(g[w], norm, S, SEED, w), range(W)))
    sums = oracle.level_sum(list(levels))
    out = oracle.qsgd_dequantize(sums, norm, S)
    return norm, levels, sums, out
