"""Binding of libgcq_ceilings.so: the benchmark's HBM ceiling kernels
(include/gcq_ceilings.h). Argument marshalling only, like the main binding:
torch tensors supply device memory and the stream.

These kernels measure what the device's HBM gives each access mix of the
hot path; they compute nothing of the method.
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Sequence

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libgcq_ceilings.so"

READ_CHUNKED, READ_TILE = 0, 1
WRITE_TILE, WRITE_STRIDE = 0, 1
DEQ_TILE, DEQ_WIDE, DEQ_BURST = 0, 1, 2

_lib = None
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i = ctypes.c_int


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "python gradient_compression_quantize_amd/build.py")
        L = ctypes.CDLL(str(LIB_PATH))
        L.gcq_ceiling_last_error.restype = ctypes.c_char_p
        L.gcq_ceiling_quantum.restype = _sz
        L.gcq_ceiling_block_words.argtypes = [_sz]
        L.gcq_ceiling_block_words.restype = _sz
        L.gcq_ceiling_read_sink_words.argtypes = [_i, _sz]
        L.gcq_ceiling_read_sink_words.restype = _sz
        L.gcq_ceiling_read.argtypes = [ctypes.POINTER(_vp), _i, _sz, _i, _vp, _sz, _vp]
        L.gcq_ceiling_write.argtypes = [_vp, _sz, _i, _vp]
        L.gcq_ceiling_compress.argtypes = [_vp, _vp, _sz, _vp, _sz, _vp]
        L.gcq_ceiling_dequant.argtypes = [ctypes.POINTER(_vp), _i, _sz, _sz, _i, _vp, _vp]
        L.gcq_ceiling_quantize.argtypes = [_vp, _sz, _vp, _vp]
        L.gcq_ceiling_ternary_quantum.restype = _sz
        L.gcq_ceiling_dequant_ternary.argtypes = [ctypes.POINTER(_vp), _i, _sz, _sz, _vp, _vp]
        L.gcq_ceiling_levelsum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp, _vp]
        L.gcq_ceiling_quantize_sum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp, _vp]
        L.gcq_ceiling_set_wg_per_cu.argtypes = [_i]
        for f in ("gcq_ceiling_set_wg_per_cu", "gcq_ceiling_read", "gcq_ceiling_write", "gcq_ceiling_compress",
                  "gcq_ceiling_dequant", "gcq_ceiling_dequant_ternary", "gcq_ceiling_quantize",
                  "gcq_ceiling_levelsum", "gcq_ceiling_quantize_sum"):
            getattr(L, f).restype = _i
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(load().gcq_ceiling_last_error().decode())


def _p(t) -> _vp:
    """Every buffer of these kernels is a contiguous device tensor of 4-byte
    elements (float32 or int32), so numel() counts 32-bit words."""
    if not t.is_cuda or not t.is_contiguous() or t.element_size() != 4:
        raise TypeError("expected a contiguous device tensor of 4-byte elements")
    return _vp(t.data_ptr())


def _arr(ts: Sequence) -> ctypes.Array:
    a = (_vp * len(ts))()
    for k, t in enumerate(ts):
        a[k] = _p(t).value
    return a


def _need(t, count: int, what: str) -> None:
    if t.numel() < count:
        raise ValueError(f"{what}: {t.numel()} elements, {count} needed")


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return _vp(s.cuda_stream)


def quantum() -> int:
    return int(load().gcq_ceiling_quantum())


def set_wg_per_cu(per_cu: int) -> None:
    """Holds later launches (all but the dequantize burst pattern) to at most
    per_cu resident workgroups per CU; 0 restores the default."""
    _check(load().gcq_ceiling_set_wg_per_cu(int(per_cu)))


def block_words(n: int) -> int:
    return int(load().gcq_ceiling_block_words(n))


def read_sink_words(nbufs: int, n: int) -> int:
    return int(load().gcq_ceiling_read_sink_words(nbufs, n))


def read(bufs: Sequence, n: int, pattern: int, sink, stream=None) -> None:
    for b in bufs:
        _need(b, n, "read buffer")
    _check(load().gcq_ceiling_read(_arr(bufs), len(bufs), n, pattern, _p(sink), sink.numel(),
                                   _stream(stream)))


def write(dst, n: int, pattern: int, stream=None) -> None:
    _need(dst, n, "write buffer")
    _check(load().gcq_ceiling_write(_p(dst), n, pattern, _stream(stream)))


def compress(a, b, n: int, words, stream=None) -> None:
    _need(a, n, "a")
    _need(b, n, "b")
    _check(load().gcq_ceiling_compress(_p(a), _p(b), n, _p(words), words.numel(),
                                       _stream(stream)))


def dequant(blocks: Sequence, n: int, pattern: int, out, stream=None) -> None:
    _need(out, n, "out")
    cap = min(b.numel() for b in blocks)
    _check(load().gcq_ceiling_dequant(_arr(blocks), len(blocks), n, cap, pattern, _p(out),
                                      _stream(stream)))


def ternary_quantum() -> int:
    return int(load().gcq_ceiling_ternary_quantum())


def dequant_ternary(blocks: Sequence, n: int, out, stream=None) -> None:
    _need(out, n, "out")
    cap = min(b.numel() for b in blocks)
    _check(load().gcq_ceiling_dequant_ternary(_arr(blocks), len(blocks), n, cap, _p(out),
                                              _stream(stream)))


def quantize(src, n: int, dst, stream=None) -> None:
    _need(src, n, "src")
    _need(dst, n // 4, "dst (words)")
    _check(load().gcq_ceiling_quantize(_p(src), n, _p(dst), _stream(stream)))


def levelsum(levels: Sequence, n: int, sums, out, stream=None) -> None:
    for q in levels:
        _need(q, n // 4, "levels (words)")
    _need(sums, n, "sums")
    _need(out, n, "out")
    _check(load().gcq_ceiling_levelsum(_arr(levels), len(levels), n, _p(sums), _p(out),
                                       _stream(stream)))


def quantize_sum(grads: Sequence, n: int, sums, out, stream=None) -> None:
    for g in grads:
        _need(g, n, "gradient")
    _need(sums, n, "sums")
    _need(out, n, "out")
    _check(load().gcq_ceiling_quantize_sum(_arr(grads), len(grads), n, _p(sums), _p(out),
                                           _stream(stream)))
