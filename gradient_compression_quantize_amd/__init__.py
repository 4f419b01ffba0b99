"""gradient_compression_quantize_amd -- gradient quantization kernels for MI355X.

Python binding of ``libgcq.so`` (HIP kernels for gfx950 behind the C ABI of
``include/gcq.h``). Each function has the name of the C entry point it calls
and only marshals arguments: torch tensors supply device memory and the
stream, and every step of the computation runs in the library's kernels.
There is no fallback: if ``libgcq.so`` is missing, ``load()`` raises.
Tensors must be contiguous, of the documented dtype, and on torch's current
device, which is where the library launches (an explicit ``stream`` must
belong to that device too); anything else is refused before the call.

Two method families (see include/gcq.h for exact semantics):
  * 2-bit threshold quantization with residual error feedback (apache MXNet
    pull request #8342): compress_2bit, decompress_2bit, decompress_2bit_sum,
    Plan2bitMulti / compress_2bit_multi, and the same codes packed five per
    byte: compress_ternary, decompress_ternary, decompress_ternary_sum;
  * QSGDMaxNorm stochastic quantization and GlobalRandK (vineeths96
    "Gradient-Compression"): qsgd_global_maxnorm (and qsgd_global_maxnorm_noalloc,
    which needs no workspace), qsgd_maxnorm_quantize,
    qsgd_dequant_sum, qsgd_quantize_sum (the W quantizes and the level sum fused),
    grandk_indices, gather_f32, and grandk_mn_step (the whole GRandK-MN step).
"""
from __future__ import annotations

import ctypes
import pathlib
from typing import Sequence

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libgcq.so"

GC_OK = 0
GC_EINVAL = -1
GC_EHIP = -2
GC_EUNSUPPORTED = -3
GC_MAX_WORKERS = 64


class GcqError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None

_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_f = ctypes.c_float
_i = ctypes.c_int


def load() -> ctypes.CDLL:
    """Load libgcq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "python gradient_compression_quantize_amd/build.py")
        _lib = _declare(ctypes.CDLL(str(LIB_PATH)))
    return _lib


def _declare(L):
    L.gc_last_error.argtypes = []
    L.gc_last_error.restype = ctypes.c_char_p
    L.gc_compressed_2bit_words.argtypes = [_sz]
    L.gc_compressed_2bit_words.restype = _sz
    L.compress_2bit.argtypes = [_vp, _vp, _sz, _f, _f, _vp, _vp]
    L.decompress_2bit.argtypes = [_vp, _sz, _vp, _i, _vp]
    L.decompress_2bit_sum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp]
    L.gc_compressed_ternary_words.argtypes = [_sz]
    L.gc_compressed_ternary_words.restype = _sz
    L.compress_ternary.argtypes = [_vp, _vp, _sz, _f, _f, _vp, _vp]
    L.decompress_ternary.argtypes = [_vp, _sz, _vp, _i, _vp]
    L.decompress_ternary_sum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp]
    L.gc_plan_2bit_multi_create.argtypes = [ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                                            ctypes.POINTER(_sz), _i, ctypes.POINTER(_vp)]
    L.gc_plan_compressed_words.argtypes = [_vp]
    L.gc_plan_compressed_words.restype = _sz
    L.gc_plan_block_offsets.argtypes = [_vp, ctypes.POINTER(_sz)]
    L.compress_2bit_multi.argtypes = [_vp, _f, _f, _vp, _vp]
    L.gc_plan_destroy.argtypes = [_vp]
    L.gc_plan_destroy.restype = None
    L.qsgd_global_maxnorm.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp,
                                      ctypes.POINTER(_sz), _vp]
    L.qsgd_global_maxnorm_noalloc.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _vp]
    L.qsgd_maxnorm_quantize.argtypes = [_vp, _sz, _vp, _i, ctypes.c_uint64, ctypes.c_uint32,
                                        _vp, _vp]
    L.qsgd_dequant_sum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _i, _vp, _vp, _vp, _sz,
                                   _vp]
    L.qsgd_quantize_sum.argtypes = [ctypes.POINTER(_vp), _i, _sz, _vp, _i, ctypes.c_uint64,
                                    _vp, _vp, _vp]
    L.grandk_indices.argtypes = [_sz, ctypes.c_uint32, ctypes.c_uint64, _vp, _vp,
                                 ctypes.POINTER(_sz), _vp]
    L.gather_f32.argtypes = [_vp, _vp, _sz, _vp, _vp]
    L.grandk_mn_step.argtypes = [ctypes.POINTER(_vp), _i, _sz, ctypes.c_uint32, ctypes.c_uint64,
                                 _i, _vp, _vp, _vp, _vp, _vp, ctypes.POINTER(_sz), _vp]
    for name in ("compress_2bit", "decompress_2bit", "decompress_2bit_sum",
                 "compress_ternary", "decompress_ternary", "decompress_ternary_sum",
                 "gc_plan_2bit_multi_create", "gc_plan_block_offsets", "compress_2bit_multi",
                 "qsgd_global_maxnorm", "qsgd_global_maxnorm_noalloc",
                 "qsgd_maxnorm_quantize", "qsgd_dequant_sum",
                 "qsgd_quantize_sum",
                 "grandk_indices", "gather_f32", "grandk_mn_step"):
        getattr(L, name).restype = _i
    return L


def last_error() -> str:
    return load().gc_last_error().decode()


def _check(rc: int) -> None:
    if rc != GC_OK:
        raise GcqError(rc, last_error())


# ---- marshalling helpers -------------------------------------------------

def _torch():
    import torch
    return torch


_gpu_present = None
_get_device = None
_raw_stream = None


def _current_device():
    """Index of torch's current device, or None when torch sees no GPU (then
    there is nothing to compare against: every call fails validation or its
    device-tensor checks first). Once torch's device state is set up, this
    reads the device straight from torch's C layer (every call of the
    binding asks once per tensor, so it is worth a few microseconds a call)."""
    global _gpu_present, _get_device, _raw_stream
    if _gpu_present is None:
        torch = _torch()
        present = bool(torch.cuda.is_available())
        if present:
            torch.cuda.current_device()  # sets up torch's device state
            _get_device = getattr(torch._C, "_cuda_getDevice", torch.cuda.current_device)
            _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _gpu_present = present
    if not _gpu_present:
        return None
    return _get_device() if _get_device is not None else _torch().cuda.current_device()


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        cur = _current_device()
        if cur is not None and _raw_stream is not None:
            # the same handle as torch.cuda.current_stream().cuda_stream,
            # without building a Stream object
            return _vp(_raw_stream(cur))
        s = torch.cuda.current_stream()
    else:
        s = stream
        dev = getattr(s, "device", None)
        cur = _current_device()
        if dev is not None and cur is not None and dev.index != cur:
            raise ValueError(f"stream is on cuda:{dev.index} but the current device is "
                             f"cuda:{cur}; the library launches on the current device")
    return _vp(s.cuda_stream)


def _refuse(t, dtype, what: str, cur) -> None:
    if not t.is_cuda:
        raise TypeError(f"{what}: expected a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{what}: expected a contiguous tensor")
    raise ValueError(f"{what}: on cuda:{t.get_device()} but the current device is "
                     f"cuda:{cur}; the library launches on the current device")


def _ptr(t, dtype, what: str, cur, k=None) -> int:
    """Device address of a contiguous tensor of the given dtype on device
    `cur` (the current device, which the library launches on; None when
    torch sees no GPU). The error names `what`, or `what[k]`."""
    if (not t.is_cuda or t.dtype != dtype or not t.is_contiguous()
            or (cur is not None and t.get_device() != cur)):
        _refuse(t, dtype, what if k is None else f"{what}[{k}]", cur)
    return t.data_ptr()


def _dev(t, dtype, what: str) -> ctypes.c_void_p:
    """Device pointer of a contiguous tensor of the given dtype on the current
    device (the device the library launches on)."""
    if t is None:
        return _vp(None)
    return _vp(_ptr(t, dtype, what, _current_device()))


def _need_norm(norm, what: str) -> None:
    """The shared max-norm is one fp32 device scalar: refuse an empty tensor
    (the kernels read element 0, and qsgd_global_maxnorm writes it)."""
    if norm is not None and norm.numel() < 1:
        raise ValueError(f"{what}: norm must hold at least one element")


def _ptr_array(ts, dtype, what: str):
    arr = (_vp * len(ts))()
    cur = _current_device()
    for k, t in enumerate(ts):
        arr[k] = None if t is None else _ptr(t, dtype, what, cur, k)
    return arr


# ---- 2-bit threshold quantization -----------------------------------------

def gc_compressed_2bit_words(n: int) -> int:
    return int(load().gc_compressed_2bit_words(n))


compressed_2bit_words = gc_compressed_2bit_words


def compress_2bit(grad, residual, neg_threshold: float, pos_threshold: float, compr,
                  stream=None) -> None:
    torch = _torch()
    n = grad.numel()
    if residual.numel() != n:
        raise ValueError("compress_2bit: grad and residual differ in size")
    if compr.numel() < gc_compressed_2bit_words(n):
        raise ValueError("compress_2bit: compr too small")
    _check(load().compress_2bit(_dev(grad, torch.float32, "grad"),
                                _dev(residual, torch.float32, "residual"), n,
                                float(neg_threshold), float(pos_threshold),
                                _dev(compr, torch.int32, "compr"), _stream(stream)))


def decompress_2bit(compr, n: int, out, accumulate: bool = False, stream=None) -> None:
    torch = _torch()
    if compr.numel() < gc_compressed_2bit_words(n) or out.numel() < n:
        raise ValueError("decompress_2bit: buffer too small")
    _check(load().decompress_2bit(_dev(compr, torch.int32, "compr"), n,
                                  _dev(out, torch.float32, "out"), int(bool(accumulate)),
                                  _stream(stream)))


def decompress_2bit_sum(comprs: Sequence, n: int, out, stream=None) -> None:
    torch = _torch()
    for c in comprs:
        if c.numel() < gc_compressed_2bit_words(n):
            raise ValueError("decompress_2bit_sum: compr too small")
    if out.numel() < n:
        raise ValueError("decompress_2bit_sum: out too small")
    arr = _ptr_array(comprs, torch.int32, "compr")
    _check(load().decompress_2bit_sum(arr, len(comprs), n, _dev(out, torch.float32, "out"),
                                      _stream(stream)))


# ---- the same codes, five per byte ------------------------------------------

def gc_compressed_ternary_words(n: int) -> int:
    return int(load().gc_compressed_ternary_words(n))


compressed_ternary_words = gc_compressed_ternary_words


def compress_ternary(grad, residual, neg_threshold: float, pos_threshold: float, compr,
                     stream=None) -> None:
    torch = _torch()
    n = grad.numel()
    if residual.numel() != n:
        raise ValueError("compress_ternary: grad and residual differ in size")
    if compr.numel() < gc_compressed_ternary_words(n):
        raise ValueError("compress_ternary: compr too small")
    _check(load().compress_ternary(_dev(grad, torch.float32, "grad"),
                                   _dev(residual, torch.float32, "residual"), n,
                                   float(neg_threshold), float(pos_threshold),
                                   _dev(compr, torch.int32, "compr"), _stream(stream)))


def decompress_ternary(compr, n: int, out, accumulate: bool = False, stream=None) -> None:
    torch = _torch()
    if compr.numel() < gc_compressed_ternary_words(n) or out.numel() < n:
        raise ValueError("decompress_ternary: buffer too small")
    _check(load().decompress_ternary(_dev(compr, torch.int32, "compr"), n,
                                     _dev(out, torch.float32, "out"), int(bool(accumulate)),
                                     _stream(stream)))


def decompress_ternary_sum(comprs: Sequence, n: int, out, stream=None) -> None:
    torch = _torch()
    for c in comprs:
        if c.numel() < gc_compressed_ternary_words(n):
            raise ValueError("decompress_ternary_sum: compr too small")
    if out.numel() < n:
        raise ValueError("decompress_ternary_sum: out too small")
    arr = _ptr_array(comprs, torch.int32, "compr")
    _check(load().decompress_ternary_sum(arr, len(comprs), n, _dev(out, torch.float32, "out"),
                                         _stream(stream)))


class Plan2bitMulti:
    """gc_plan_2bit_multi_create / compress_2bit_multi / gc_plan_destroy.
    Holds references to the tensors so their memory outlives the plan."""

    def __init__(self, grads: Sequence, residuals: Sequence):
        torch = _torch()
        if len(grads) != len(residuals) or not grads:
            raise ValueError("Plan2bitMulti: need matching, non-empty tensor lists")
        T = len(grads)
        ns = (_sz * T)(*[g.numel() for g in grads])
        for g, r in zip(grads, residuals):
            if g.numel() != r.numel():
                raise ValueError("Plan2bitMulti: grad and residual differ in size")
        self._keep = (list(grads), list(residuals))
        self.sizes = [g.numel() for g in grads]
        handle = _vp()
        _check(load().gc_plan_2bit_multi_create(_ptr_array(grads, torch.float32, "grads"),
                                                _ptr_array(residuals, torch.float32, "residuals"),
                                                ns, T, ctypes.byref(handle)))
        self._handle = handle

    @property
    def compressed_words(self) -> int:
        return int(load().gc_plan_compressed_words(self._handle))

    def block_offsets(self) -> list[int]:
        T = len(self.sizes)
        out = (_sz * T)()
        _check(load().gc_plan_block_offsets(self._handle, out))
        return list(out)

    def compress(self, neg_threshold: float, pos_threshold: float, compr_base,
                 stream=None) -> None:
        torch = _torch()
        if compr_base.numel() < self.compressed_words:
            raise ValueError("compress_2bit_multi: compr_base too small")
        _check(load().compress_2bit_multi(self._handle, float(neg_threshold),
                                          float(pos_threshold),
                                          _dev(compr_base, torch.int32, "compr_base"),
                                          _stream(stream)))

    def destroy(self) -> None:
        if getattr(self, "_handle", None) is not None and self._handle.value:
            load().gc_plan_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def compress_2bit_multi(plan: Plan2bitMulti, neg_threshold: float, pos_threshold: float,
                        compr_base, stream=None) -> None:
    plan.compress(neg_threshold, pos_threshold, compr_base, stream)


# ---- QSGDMaxNorm ----------------------------------------------------------

def qsgd_maxnorm_ws_bytes(W: int, n: int) -> int:
    size = _sz(0)
    _check(load().qsgd_global_maxnorm(None, W, n, None, None, ctypes.byref(size), None))
    return int(size.value)


def qsgd_global_maxnorm(grads: Sequence, norm, ws, stream=None) -> None:
    """norm: 1-element float32 device tensor; ws: uint8 device tensor of at
    least qsgd_maxnorm_ws_bytes(W, n) bytes."""
    torch = _torch()
    n = grads[0].numel()
    for g in grads:
        if g.numel() != n:
            raise ValueError("qsgd_global_maxnorm: gradients differ in size")
    _need_norm(norm, "qsgd_global_maxnorm")
    size = _sz(ws.numel())
    _check(load().qsgd_global_maxnorm(_ptr_array(grads, torch.float32, "grads"), len(grads), n,
                                      _dev(norm, torch.float32, "norm"),
                                      _dev(ws, torch.uint8, "ws"), ctypes.byref(size),
                                      _stream(stream)))


def qsgd_global_maxnorm_noalloc(grads: Sequence, norm, stream=None) -> None:
    """qsgd_global_maxnorm without a workspace: the partial maxima go to the
    library's fixed device array. Calls that overlap on one device race."""
    torch = _torch()
    n = grads[0].numel()
    for g in grads:
        if g.numel() != n:
            raise ValueError("qsgd_global_maxnorm_noalloc: gradients differ in size")
    _need_norm(norm, "qsgd_global_maxnorm_noalloc")
    _check(load().qsgd_global_maxnorm_noalloc(_ptr_array(grads, torch.float32, "grads"),
                                              len(grads), n, _dev(norm, torch.float32, "norm"),
                                              _stream(stream)))


def qsgd_maxnorm_quantize(grad, norm, s: int, seed: int, worker: int, levels,
                          stream=None) -> None:
    torch = _torch()
    n = grad.numel()
    if levels.numel() < n:
        raise ValueError("qsgd_maxnorm_quantize: levels too small")
    _need_norm(norm, "qsgd_maxnorm_quantize")
    _check(load().qsgd_maxnorm_quantize(_dev(grad, torch.float32, "grad"), n,
                                        _dev(norm, torch.float32, "norm"), int(s), int(seed),
                                        int(worker), _dev(levels, torch.int8, "levels"),
                                        _stream(stream)))


def qsgd_dequant_sum(levels: Sequence, norm, s: int, out, sums=None, scatter_idx=None,
                     dense_n: int = 0, stream=None) -> None:
    torch = _torch()
    n = levels[0].numel()
    for q in levels:
        if q.numel() != n:
            raise ValueError("qsgd_dequant_sum: level arrays differ in size")
    if scatter_idx is None:
        if out.numel() < n or (sums is not None and sums.numel() < n):
            raise ValueError("qsgd_dequant_sum: output too small")
    else:
        if scatter_idx.numel() != n or out.numel() < dense_n:
            raise ValueError("qsgd_dequant_sum: scatter_idx / out size mismatch")
        if sums is not None and sums.numel() < n:
            raise ValueError("qsgd_dequant_sum: sums too small")
    _need_norm(norm, "qsgd_dequant_sum")
    _check(load().qsgd_dequant_sum(_ptr_array(levels, torch.int8, "levels"), len(levels), n,
                                   _dev(norm, torch.float32, "norm"), int(s),
                                   _dev(sums, torch.int32, "sums"),
                                   _dev(out, torch.float32, "out"),
                                   _dev(scatter_idx, torch.int32, "scatter_idx"),
                                   int(dense_n), _stream(stream)))


# ---- GlobalRandK ------------------------------------------------------------

def qsgd_quantize_sum(grads: Sequence, norm, s: int, seed: int, out, sums=None,
                      stream=None) -> None:
    torch = _torch()
    n = grads[0].numel()
    if any(g.numel() != n for g in grads):
        raise ValueError("qsgd_quantize_sum: gradients differ in size")
    if out.numel() < n or (sums is not None and sums.numel() < n):
        raise ValueError("qsgd_quantize_sum: out or sums too small")
    _need_norm(norm, "qsgd_quantize_sum")
    arr = _ptr_array(grads, torch.float32, "grads")
    _check(load().qsgd_quantize_sum(arr, len(grads), n, _dev(norm, torch.float32, "norm"),
                                    int(s), int(seed) & (2 ** 64 - 1),
                                    _dev(sums, torch.int32, "sums"),
                                    _dev(out, torch.float32, "out"), _stream(stream)))


def grandk_ws_bytes(n: int, K: int) -> int:
    size = _sz(0)
    _check(load().grandk_indices(n, K, 0, None, None, ctypes.byref(size), None))
    return int(size.value)


def grandk_indices(n: int, K: int, seed: int, idx, ws, stream=None) -> None:
    """idx: int32 device tensor of K elements (holding uint32 values < 2^31
    for any n a torch int32 tensor can index); ws: uint8 device tensor."""
    torch = _torch()
    if idx.numel() < K:
        raise ValueError("grandk_indices: idx too small")
    size = _sz(ws.numel())
    _check(load().grandk_indices(n, K, int(seed), _dev(idx, torch.int32, "idx"),
                                 _dev(ws, torch.uint8, "ws"), ctypes.byref(size),
                                 _stream(stream)))


def gather_f32(x, idx, out, stream=None) -> None:
    torch = _torch()
    K = idx.numel()
    if out.numel() < K:
        raise ValueError("gather_f32: out too small")
    _check(load().gather_f32(_dev(x, torch.float32, "x"), _dev(idx, torch.int32, "idx"), K,
                             _dev(out, torch.float32, "out"), _stream(stream)))


def grandk_mn_step_ws_bytes(W: int, n: int, K: int) -> int:
    size = _sz(0)
    arr = (_vp * W)()
    _check(load().grandk_mn_step(arr, W, n, K, 0, 7, None, None, None, None, None,
                                 ctypes.byref(size), None))
    return size.value


def grandk_mn_step(grads: Sequence, K: int, seed: int, s: int, idx, dense, ws, sums=None,
                   norm=None, stream=None) -> None:
    torch = _torch()
    n = grads[0].numel()
    if any(g.numel() != n for g in grads):
        raise ValueError("grandk_mn_step: gradients differ in size")
    if idx.numel() < K or dense.numel() < n or (sums is not None and sums.numel() < K):
        raise ValueError("grandk_mn_step: idx, sums or dense too small")
    _need_norm(norm, "grandk_mn_step")
    arr = _ptr_array(grads, torch.float32, "grads")
    size = _sz(ws.numel() * ws.element_size())
    _check(load().grandk_mn_step(arr, len(grads), n, K, int(seed) & (2 ** 64 - 1), int(s),
                                 _dev(idx, torch.int32, "idx"), _dev(sums, torch.int32, "sums"),
                                 _dev(dense, torch.float32, "dense"),
                                 _dev(norm, torch.float32, "norm"), _dev(ws, torch.uint8, "ws"),
                                 ctypes.byref(size), _stream(stream)))
