"""CPU oracle for the gradient-quantization hot path -- TEST INFRASTRUCTURE ONLY.

A thin numpy wrapper over ``liboracle.so`` (plain single-threaded C, built
from ``oracle.c`` with gcc). Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the HIP library and its
Python binding never do, and the two share no code.

Each function here only marshals numpy arrays; the arithmetic lives in
``oracle.c``, which cites the passages it follows.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
SOURCE = _HERE / "oracle.c"
LIB_PATH = _HERE / "liboracle.so"

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-msse2", "-mfpmath=sse", "-Wall", "-Wextra", "-Werror",
          "-shared", "-fPIC"]


def build(verbose: bool = False) -> pathlib.Path:
    """Compile liboracle.so with gcc (always recompiles)."""
    tmp = LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", *CFLAGS, str(SOURCE), "-o", str(tmp), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it first only if it does not exist.

    GCQ_ORACLE_LIB may name another build of oracle.c; the mutation test uses
    it to run the pins against copies with planted mistakes."""
    global _lib
    if _lib is None:
        override = os.environ.get("GCQ_ORACLE_LIB")
        if override:
            _lib = _declare(ctypes.CDLL(override))
        else:
            if not LIB_PATH.exists():
                build()
            _lib = _declare(ctypes.CDLL(str(LIB_PATH)))
    return _lib


_f32p = ctypes.POINTER(ctypes.c_float)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_i8p = ctypes.POINTER(ctypes.c_int8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_sz = ctypes.c_size_t


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    L.oracle_compressed_2bit_words.argtypes = [_sz]
    L.oracle_compressed_2bit_words.restype = _sz
    L.oracle_quantize_2bit.argtypes = [_f32p, _f32p, _sz, ctypes.c_float,
                                       ctypes.c_float, _u32p]
    L.oracle_quantize_2bit.restype = None
    L.oracle_dequantize_2bit.argtypes = [_u32p, _sz, _f32p]
    L.oracle_dequantize_2bit.restype = None
    L.oracle_dequantize_2bit_sum.argtypes = [ctypes.POINTER(_u32p), ctypes.c_int,
                                             _sz, _f32p]
    L.oracle_dequantize_2bit_sum.restype = None
    L.oracle_compressed_ternary_words.argtypes = [_sz]
    L.oracle_compressed_ternary_words.restype = _sz
    L.oracle_quantize_ternary.argtypes = [_f32p, _f32p, _sz, ctypes.c_float,
                                          ctypes.c_float, _u32p]
    L.oracle_quantize_ternary.restype = None
    L.oracle_dequantize_ternary.argtypes = [_u32p, _sz, _f32p]
    L.oracle_dequantize_ternary.restype = None
    L.oracle_dequantize_ternary_sum.argtypes = [ctypes.POINTER(_u32p), ctypes.c_int,
                                                _sz, _f32p]
    L.oracle_dequantize_ternary_sum.restype = None
    L.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    L.oracle_philox4x32_10.restype = None
    L.oracle_uniform24.argtypes = [ctypes.c_uint32]
    L.oracle_uniform24.restype = ctypes.c_float
    L.oracle_stochastic_level.argtypes = [ctypes.c_float, ctypes.c_float]
    L.oracle_stochastic_level.restype = ctypes.c_int
    L.oracle_maxnorm.argtypes = [ctypes.POINTER(_f32p), ctypes.c_int, _sz]
    L.oracle_maxnorm.restype = ctypes.c_float
    L.oracle_qsgd_quantize.argtypes = [_f32p, _sz, ctypes.c_float, ctypes.c_int,
                                       ctypes.c_uint64, ctypes.c_uint32, _i8p]
    L.oracle_qsgd_quantize.restype = None
    L.oracle_qsgd_quantize_at.argtypes = [_f32p, _u64p, _sz, ctypes.c_float,
                                          ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint32, _i8p]
    L.oracle_qsgd_quantize_at.restype = None
    L.oracle_level_sum.argtypes = [ctypes.POINTER(_i8p), ctypes.c_int, _sz, _i32p]
    L.oracle_level_sum.restype = None
    L.oracle_qsgd_dequantize.argtypes = [_i32p, _sz, ctypes.c_float, ctypes.c_int,
                                         _f32p]
    L.oracle_qsgd_dequantize.restype = None
    L.oracle_randk_indices.argtypes = [_sz, ctypes.c_uint32, ctypes.c_uint64, _u32p]
    L.oracle_randk_indices.restype = ctypes.c_int
    L.oracle_gather.argtypes = [_f32p, _u32p, _sz, _f32p]
    L.oracle_gather.restype = None
    L.oracle_scatter_dense.argtypes = [_f32p, _u32p, _sz, _sz, _f32p]
    L.oracle_scatter_dense.restype = None
    return L


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as(a, dtype) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------- 2-bit ----

def compressed_2bit_words(n: int) -> int:
    return int(lib().oracle_compressed_2bit_words(n))


def quantize_2bit(grad: np.ndarray, residual: np.ndarray, neg_threshold: float,
                  pos_threshold: float) -> np.ndarray:
    """Returns the compressed block; `residual` (float32, contiguous) is
    updated in place."""
    grad = _as(grad, np.float32)
    if residual.dtype != np.float32 or not residual.flags["C_CONTIGUOUS"]:
        raise TypeError("residual must be a contiguous float32 array")
    n = grad.size
    assert residual.size == n
    compr = np.empty(compressed_2bit_words(n), dtype=np.uint32)
    lib().oracle_quantize_2bit(_ptr(grad, ctypes.c_float),
                               _ptr(residual, ctypes.c_float), n,
                               float(neg_threshold), float(pos_threshold),
                               _ptr(compr, ctypes.c_uint32))
    return compr


def dequantize_2bit(compr: np.ndarray, n: int) -> np.ndarray:
    compr = _as(compr, np.uint32)
    assert compr.size == compressed_2bit_words(n)
    out = np.empty(n, dtype=np.float32)
    lib().oracle_dequantize_2bit(_ptr(compr, ctypes.c_uint32), n,
                                 _ptr(out, ctypes.c_float))
    return out


def dequantize_2bit_sum(comprs, n: int) -> np.ndarray:
    comprs = [_as(c, np.uint32) for c in comprs]
    W = len(comprs)
    for c in comprs:
        assert c.size == compressed_2bit_words(n)
    arr = (_u32p * W)(*[_ptr(c, ctypes.c_uint32) for c in comprs])
    out = np.empty(n, dtype=np.float32)
    lib().oracle_dequantize_2bit_sum(arr, W, n, _ptr(out, ctypes.c_float))
    return out


# -------------------------------------------------------------- ternary ----

def compressed_ternary_words(n: int) -> int:
    return int(lib().oracle_compressed_ternary_words(n))


def quantize_ternary(grad: np.ndarray, residual: np.ndarray, neg_threshold: float,
                     pos_threshold: float) -> np.ndarray:
    grad = _as(grad, np.float32)
    if residual.dtype != np.float32 or not residual.flags["C_CONTIGUOUS"]:
        raise TypeError("residual must be a contiguous float32 array")
    n = grad.size
    assert residual.size == n
    compr = np.empty(compressed_ternary_words(n), dtype=np.uint32)
    lib().oracle_quantize_ternary(_ptr(grad, ctypes.c_float), _ptr(residual, ctypes.c_float),
                                  n, float(neg_threshold), float(pos_threshold),
                                  _ptr(compr, ctypes.c_uint32))
    return compr


def dequantize_ternary(compr: np.ndarray, n: int) -> np.ndarray:
    compr = _as(compr, np.uint32)
    assert compr.size == compressed_ternary_words(n)
    out = np.empty(n, dtype=np.float32)
    lib().oracle_dequantize_ternary(_ptr(compr, ctypes.c_uint32), n, _ptr(out, ctypes.c_float))
    return out


def dequantize_ternary_sum(comprs, n: int) -> np.ndarray:
    comprs = [_as(c, np.uint32) for c in comprs]
    for c in comprs:
        assert c.size == compressed_ternary_words(n)
    arr = (_u32p * len(comprs))(*[_ptr(c, ctypes.c_uint32) for c in comprs])
    out = np.empty(n, dtype=np.float32)
    lib().oracle_dequantize_ternary_sum(arr, len(comprs), n, _ptr(out, ctypes.c_float))
    return out


# --------------------------------------------------------------- Philox ----

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.empty(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32),
                               _ptr(out, ctypes.c_uint32))
    return out


# ----------------------------------------------------------------- QSGD ----

def uniform24(r: int) -> float:
    return float(lib().oracle_uniform24(int(r)))


def stochastic_level(x: float, u: float) -> int:
    return int(lib().oracle_stochastic_level(float(x), float(u)))


def maxnorm(grads) -> np.float32:
    grads = [_as(g, np.float32) for g in grads]
    n = grads[0].size
    for g in grads:
        assert g.size == n
    arr = (_f32p * len(grads))(*[_ptr(g, ctypes.c_float) for g in grads])
    return np.float32(lib().oracle_maxnorm(arr, len(grads), n))


def qsgd_quantize(grad: np.ndarray, norm, s: int, seed: int, worker: int) -> np.ndarray:
    grad = _as(grad, np.float32)
    out = np.empty(grad.size, dtype=np.int8)
    lib().oracle_qsgd_quantize(_ptr(grad, ctypes.c_float), grad.size, float(norm),
                               int(s), int(seed), int(worker), _ptr(out, ctypes.c_int8))
    return out


def qsgd_quantize_at(values: np.ndarray, index: np.ndarray, norm, s: int,
                     seed: int, worker: int) -> np.ndarray:
    values = _as(values, np.float32)
    index = _as(index, np.uint64)
    assert values.size == index.size
    out = np.empty(values.size, dtype=np.int8)
    lib().oracle_qsgd_quantize_at(_ptr(values, ctypes.c_float),
                                  _ptr(index, ctypes.c_uint64), values.size,
                                  float(norm), int(s), int(seed), int(worker),
                                  _ptr(out, ctypes.c_int8))
    return out


def level_sum(levels) -> np.ndarray:
    levels = [_as(q, np.int8) for q in levels]
    n = levels[0].size
    arr = (_i8p * len(levels))(*[_ptr(q, ctypes.c_int8) for q in levels])
    out = np.empty(n, dtype=np.int32)
    lib().oracle_level_sum(arr, len(levels), n, _ptr(out, ctypes.c_int32))
    return out


def qsgd_dequantize(sums: np.ndarray, norm, s: int) -> np.ndarray:
    sums = _as(sums, np.int32)
    out = np.empty(sums.size, dtype=np.float32)
    lib().oracle_qsgd_dequantize(_ptr(sums, ctypes.c_int32), sums.size, float(norm),
                                 int(s), _ptr(out, ctypes.c_float))
    return out


# -------------------------------------------------------------- rand-K ----

def randk_indices(n: int, K: int, seed: int) -> np.ndarray:
    idx = np.empty(K, dtype=np.uint32)
    rc = lib().oracle_randk_indices(n, K, int(seed), _ptr(idx, ctypes.c_uint32))
    if rc != 0:
        raise ValueError(f"oracle_randk_indices(n={n}, K={K}) failed: {rc}")
    return idx


def gather(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    x = _as(x, np.float32)
    idx = _as(idx, np.uint32)
    assert idx.size == 0 or int(idx.max()) < x.size
    out = np.empty(idx.size, dtype=np.float32)
    lib().oracle_gather(_ptr(x, ctypes.c_float), _ptr(idx, ctypes.c_uint32),
                        idx.size, _ptr(out, ctypes.c_float))
    return out


def scatter_dense(vals: np.ndarray, idx: np.ndarray, dense_n: int) -> np.ndarray:
    vals = _as(vals, np.float32)
    idx = _as(idx, np.uint32)
    assert vals.size == idx.size
    assert idx.size == 0 or int(idx.max()) < dense_n
    out = np.empty(dense_n, dtype=np.float32)
    lib().oracle_scatter_dense(_ptr(vals, ctypes.c_float), _ptr(idx, ctypes.c_uint32),
                               idx.size, dense_n, _ptr(out, ctypes.c_float))
    return out
