"""The C-ABI boundary, without a GPU: libgcq.so loads, exports every entry
point include/gcq.h declares (and nothing else), sizes its outputs like the
oracle, and rejects bad arguments on the host before enqueuing anything.

Only host-side paths are called here: validation failures and workspace-size
queries return before any HIP call.
"""
import ctypes
import math
import pathlib
import re
import subprocess

import pytest

import gradient_compression_quantize_amd as gcq
import oracle

ROOT = pathlib.Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "gcq.h"

NULL = None
FAKE = 0x10000  # a 16-byte-aligned address that is never dereferenced


def declared_functions(header: pathlib.Path = HEADER) -> set[str]:
    text = header.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return set(names)


@pytest.fixture(scope="module")
def lib():
    if not gcq.LIB_PATH.exists():
        pytest.fail("libgcq.so is not built (python gradient_compression_quantize_amd/build.py)")
    return gcq.load()


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ("compress_2bit", "decompress_2bit", "decompress_2bit_sum",
                 "qsgd_maxnorm_quantize", "qsgd_dequant_sum", "qsgd_global_maxnorm",
                 "grandk_indices", "gather_f32", "compress_2bit_multi",
                 "gc_plan_2bit_multi_create", "gc_plan_destroy", "gc_compressed_2bit_words",
                 "gc_plan_compressed_words", "gc_plan_block_offsets", "gc_last_error",
                 "gc_compressed_ternary_words", "compress_ternary", "decompress_ternary",
                 "decompress_ternary_sum", "qsgd_quantize_sum", "grandk_mn_step"):
        assert must in names, must


def test_library_exports_exactly_the_declared_symbols(lib):
    names = declared_functions()
    for name in names:
        assert hasattr(lib, name), f"{name} declared in gcq.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", str(gcq.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == names, (exported - names, names - exported)


def test_ceilings_library_exports_exactly_its_header_and_refuses_bad_sizes():
    """libgcq_ceilings.so (the benchmark's streaming kernels) against
    include/gcq_ceilings.h, and its host-side refusals, which return before
    any HIP call."""
    from gradient_compression_quantize_amd import ceilings as cl
    if not cl.LIB_PATH.exists():
        pytest.fail("libgcq_ceilings.so is not built (python gradient_compression_quantize_amd/build.py)")
    names = declared_functions(ROOT / "include" / "gcq_ceilings.h")
    assert {"gcq_ceiling_read", "gcq_ceiling_write", "gcq_ceiling_compress", "gcq_ceiling_dequant",
            "gcq_ceiling_dequant_ternary", "gcq_ceiling_quantize", "gcq_ceiling_levelsum",
            "gcq_ceiling_quantize_sum"} <= names
    out = subprocess.run(["nm", "-D", "--defined-only", str(cl.LIB_PATH)],
                         capture_output=True, text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == names, (exported - names, names - exported)
    L = cl.load()
    q = cl.quantum()
    assert q == 16384 and cl.ternary_quantum() == 81920
    assert cl.block_words(q) == 3 + q // 16 + 4
    arr = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    # sizes off the quantum, the wrong worker count and misaligned buffers
    assert L.gcq_ceiling_write(FAKE, q + 1, 0, None) == -1
    assert "bad arguments" in L.gcq_ceiling_last_error().decode()
    assert L.gcq_ceiling_quantize_sum(arr, 7, q, FAKE, FAKE, None) == -1
    assert L.gcq_ceiling_quantize_sum(arr, 8, q, FAKE + 4, FAKE, None) == -1
    assert L.gcq_ceiling_levelsum(arr, 8, q - 16, FAKE, FAKE, None) == -1
    assert L.gcq_ceiling_dequant(arr, 8, q, 16, 0, FAKE, None) == -1
    assert L.gcq_ceiling_compress(FAKE, FAKE, q, FAKE, 16, None) == -1
    # the occupancy cap: negative counts are refused, 0..n accepted (host state only)
    assert L.gcq_ceiling_set_wg_per_cu(-1) == -1
    assert "per_cu" in L.gcq_ceiling_last_error().decode()
    assert L.gcq_ceiling_set_wg_per_cu(3) == 0 and L.gcq_ceiling_set_wg_per_cu(0) == 0


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 4096, 25_557_032, 2 ** 33 + 5, 2 ** 64 - 1])
def test_compressed_words_matches_oracle(lib, n):
    assert lib.gc_compressed_2bit_words(n) == 3 + (n + 15) // 16
    if n < 10 ** 8:
        assert lib.gc_compressed_2bit_words(n) == oracle.compressed_2bit_words(n)


@pytest.mark.parametrize("n", [0, 1, 19, 20, 21, 1280, 25_557_032, 2 ** 33 + 5, 2 ** 64 - 1])
def test_compressed_ternary_words_matches_oracle(lib, n):
    assert lib.gc_compressed_ternary_words(n) == 3 + (n + 19) // 20
    if n < 10 ** 8:
        assert lib.gc_compressed_ternary_words(n) == oracle.compressed_ternary_words(n)


def _rc_compress(lib, grad, res, n, neg, pos, compr):
    return lib.compress_2bit(grad, res, n, neg, pos, compr, None)


@pytest.mark.parametrize("neg,pos", [(0.0, 1.0), (-1.0, 0.0), (1.0, 2.0), (-2.0, -1.0),
                                     (-math.inf, 1.0), (-1.0, math.inf), (math.nan, 1.0),
                                     (-1.0, math.nan)])
def test_compress_rejects_bad_thresholds(lib, neg, pos):
    assert _rc_compress(lib, FAKE, FAKE, 16, neg, pos, FAKE) == gcq.GC_EINVAL
    assert b"threshold" in lib.gc_last_error()
    assert lib.compress_2bit_multi(FAKE, neg, pos, FAKE, None) == gcq.GC_EINVAL
    assert lib.compress_ternary(FAKE, FAKE, 16, neg, pos, FAKE, None) == gcq.GC_EINVAL


def test_compress_rejects_null_and_misaligned(lib):
    assert _rc_compress(lib, FAKE, FAKE, 16, -1.0, 1.0, NULL) == gcq.GC_EINVAL
    assert _rc_compress(lib, NULL, FAKE, 16, -1.0, 1.0, FAKE) == gcq.GC_EINVAL
    assert _rc_compress(lib, FAKE, NULL, 16, -1.0, 1.0, FAKE) == gcq.GC_EINVAL
    assert _rc_compress(lib, FAKE + 2, FAKE, 16, -1.0, 1.0, FAKE) == gcq.GC_EINVAL
    assert _rc_compress(lib, FAKE, FAKE, 16, -1.0, 1.0, FAKE + 1) == gcq.GC_EINVAL


def test_decompress_rejects_bad_arguments(lib):
    assert lib.decompress_2bit(NULL, 16, FAKE, 0, None) == gcq.GC_EINVAL
    assert lib.decompress_2bit(FAKE, 16, NULL, 0, None) == gcq.GC_EINVAL
    assert lib.decompress_2bit(FAKE, 16, FAKE, 2, None) == gcq.GC_EINVAL
    arr = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert lib.decompress_2bit_sum(arr, 0, 16, FAKE, None) == gcq.GC_EINVAL
    assert lib.decompress_2bit_sum(arr, 65, 16, FAKE, None) == gcq.GC_EINVAL
    arr[1] = None
    assert lib.decompress_2bit_sum(arr, 2, 16, FAKE, None) == gcq.GC_EINVAL


def test_ternary_rejects_null_and_misaligned(lib):
    for args in ((FAKE, FAKE, 16, -1.0, 1.0, NULL), (NULL, FAKE, 16, -1.0, 1.0, FAKE),
                 (FAKE, NULL, 16, -1.0, 1.0, FAKE), (FAKE + 2, FAKE, 16, -1.0, 1.0, FAKE),
                 (FAKE, FAKE, 16, -1.0, 1.0, FAKE + 1)):
        assert lib.compress_ternary(*args, None) == gcq.GC_EINVAL
    assert lib.decompress_ternary(NULL, 16, FAKE, 0, None) == gcq.GC_EINVAL
    assert lib.decompress_ternary(FAKE, 16, NULL, 0, None) == gcq.GC_EINVAL
    assert lib.decompress_ternary(FAKE, 16, FAKE, 2, None) == gcq.GC_EINVAL
    arr = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    assert lib.decompress_ternary_sum(arr, 0, 16, FAKE, None) == gcq.GC_EINVAL
    assert lib.decompress_ternary_sum(arr, 65, 16, FAKE, None) == gcq.GC_EINVAL
    arr[1] = None
    assert lib.decompress_ternary_sum(arr, 2, 16, FAKE, None) == gcq.GC_EINVAL
    assert b"decompress_ternary_sum" in lib.gc_last_error()


def test_qsgd_rejects_bad_arguments(lib):
    for s in (0, 128, -1):
        assert lib.qsgd_maxnorm_quantize(FAKE, 16, FAKE, s, 0, 0, FAKE, None) == gcq.GC_EINVAL
    assert lib.qsgd_maxnorm_quantize(FAKE, 16, NULL, 7, 0, 0, FAKE, None) == gcq.GC_EINVAL
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    for W in (0, 65):
        assert lib.qsgd_dequant_sum(arr, W, 16, FAKE, 7, NULL, FAKE, NULL, 0, None) == gcq.GC_EINVAL
    assert lib.qsgd_dequant_sum(arr, 2, 16, FAKE, 0, NULL, FAKE, NULL, 0, None) == gcq.GC_EINVAL
    # more scattered values than the dense output holds
    assert lib.qsgd_dequant_sum(arr, 2, 16, FAKE, 7, NULL, FAKE, FAKE, 8, None) == gcq.GC_EINVAL


def test_quantize_sum_rejects_bad_arguments(lib):
    arr = (ctypes.c_void_p * 65)(*([FAKE] * 65))
    for W in (0, 65):
        assert lib.qsgd_quantize_sum(arr, W, 16, FAKE, 7, 0, NULL, FAKE, None) == gcq.GC_EINVAL
    for s in (0, 128):
        assert lib.qsgd_quantize_sum(arr, 2, 16, FAKE, s, 0, NULL, FAKE, None) == gcq.GC_EINVAL
    assert lib.qsgd_quantize_sum(arr, 2, 16, NULL, 7, 0, NULL, FAKE, None) == gcq.GC_EINVAL
    assert lib.qsgd_quantize_sum(arr, 2, 16, FAKE, 7, 0, NULL, NULL, None) == gcq.GC_EINVAL
    assert lib.qsgd_quantize_sum(arr, 2, 16, FAKE, 7, 0, FAKE + 2, FAKE, None) == gcq.GC_EINVAL
    arr[1] = FAKE + 2
    assert lib.qsgd_quantize_sum(arr, 2, 16, FAKE, 7, 0, NULL, FAKE, None) == gcq.GC_EINVAL
    arr[1] = None
    assert lib.qsgd_quantize_sum(arr, 2, 16, FAKE, 7, 0, NULL, FAKE, None) == gcq.GC_EINVAL
    assert b"qsgd_quantize_sum" in lib.gc_last_error()


def test_workspace_queries(lib):
    size = ctypes.c_size_t(0)
    assert lib.qsgd_global_maxnorm(None, 8, 138_357_544, None, None, ctypes.byref(size), None) == 0
    assert 0 < size.value <= 8 * 4096 * 4
    small = ctypes.c_size_t(size.value - 4)
    arr = (ctypes.c_void_p * 8)(*([FAKE] * 8))
    assert lib.qsgd_global_maxnorm(arr, 8, 138_357_544, FAKE, FAKE, ctypes.byref(small),
                                   None) == gcq.GC_EINVAL
    assert lib.grandk_indices(25_557_032, 10_000, 0, None, None, ctypes.byref(size), None) == 0
    assert size.value == 4 * (32768 + 2 * 10_000)
    assert lib.grandk_indices(10, 11, 0, None, None, ctypes.byref(size), None) == gcq.GC_EINVAL
    assert lib.grandk_indices(2 ** 32 + 1, 1, 0, None, None, ctypes.byref(size), None) == gcq.GC_EINVAL


def test_grandk_mn_step_workspace_and_validation(lib):
    size = ctypes.c_size_t(0)
    arr = (ctypes.c_void_p * 64)(*([FAKE] * 64))
    assert lib.grandk_mn_step(arr, 8, 25_557_032, 10_000, 0, 7, None, None, None, None, None,
                              ctypes.byref(size), None) == 0
    # gathered values (8 x 10000 fp32) + partial maxima; the draw uses LDS
    assert 8 * 10_000 * 4 <= size.value <= 8 * 10_000 * 4 + 8192
    big = ctypes.c_size_t(0)
    assert lib.grandk_mn_step(arr, 2, 10 ** 6, 20_000, 0, 7, None, None, None, None, None,
                              ctypes.byref(big), None) == 0
    assert big.value >= 2 * 20_000 * 4 + 4 * (65536 + 2 * 20_000)
    bad = [(0, 100, 10, 7), (65, 100, 10, 7), (2, 100, 101, 7), (2, 0, 0, 7), (2, 100, 10, 0),
           (2, 100, 10, 128), (2, 2 ** 32 + 1, 10, 7)]
    for W, n, K, s in bad:
        assert lib.grandk_mn_step(arr, W, n, K, 0, s, None, None, None, None, None,
                                  ctypes.byref(size), None) == gcq.GC_EINVAL, (W, n, K, s)
    small = ctypes.c_size_t(16)
    assert lib.grandk_mn_step(arr, 2, 100, 10, 0, 7, FAKE, NULL, FAKE, NULL, FAKE,
                              ctypes.byref(small), None) == gcq.GC_EINVAL
    assert lib.grandk_mn_step(arr, 2, 100, 10, 0, 7, FAKE, NULL, FAKE, NULL, NULL, NULL,
                              None) == gcq.GC_EINVAL


def test_plan_rejects_bad_arguments(lib):
    handle = ctypes.c_void_p()
    ns = (ctypes.c_size_t * 1)(16)
    ptrs = (ctypes.c_void_p * 1)(None)
    assert lib.gc_plan_2bit_multi_create(ptrs, ptrs, ns, 1, ctypes.byref(handle)) == gcq.GC_EINVAL
    assert lib.gc_plan_2bit_multi_create(ptrs, ptrs, ns, 0, ctypes.byref(handle)) == gcq.GC_EINVAL
    assert handle.value is None


def test_error_message_is_per_thread(lib):
    """gc_last_error() reports the calling thread's own last failure: two
    threads fail different calls in lockstep and each reads its own message
    (ctypes drops the GIL inside the calls, so they run concurrently)."""
    import threading

    rounds = 2000
    barrier = threading.Barrier(2, timeout=30)
    errors = []
    arr = (ctypes.c_void_p * 64)(*([FAKE] * 64))

    def run(name, call, code, text):
        try:
            for _ in range(rounds):
                barrier.wait()
                if call() != code:
                    errors.append(f"{name}: wrong return code")
                barrier.wait()
                if text not in lib.gc_last_error():
                    errors.append(f"{name}: message of another thread")
        except Exception as e:  # a failing thread must not leave the other waiting
            errors.append(f"{name}: {e!r}")
            barrier.abort()

    threads = [
        threading.Thread(target=run, args=(
            "compress", lambda: _rc_compress(lib, FAKE, FAKE, 16, 1.0, -1.0, FAKE),
            gcq.GC_EINVAL, b"threshold")),
        threading.Thread(target=run, args=(
            "sum", lambda: lib.decompress_2bit_sum(arr, 0, 16, FAKE, None),
            gcq.GC_EINVAL, b"W must be")),
    ]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors[:3]
    # a successful call clears the calling thread's message
    size = ctypes.c_size_t(0)
    assert lib.grandk_indices(100, 10, 0, NULL, NULL, ctypes.byref(size), None) == gcq.GC_OK
    assert lib.gc_last_error() == b""


def test_abi_client_finds_its_libraries_relative_to_itself():
    """tests/_bin/abi_client (the C-ABI client the GPU suite runs) needs
    libgcq.so and liboracle.so by name and finds them through a RUNPATH
    relative to its own location, so the built tree can move to another
    machine."""
    import abi_client_build as acb
    if not acb.BIN.exists():
        pytest.fail(f"{acb.BIN} is not built: run python tests/abi_client_build.py (or build())")
    out = subprocess.run(["readelf", "-d", str(acb.BIN)], capture_output=True, text=True,
                         check=True).stdout
    needed = set(re.findall(r"\(NEEDED\)\s+Shared library: \[([^\]]+)\]", out))
    assert {"libgcq.so", "liboracle.so"} <= needed
    runpath = re.search(r"\((?:RUNPATH|RPATH)\)\s+Library (?:runpath|rpath): \[([^\]]+)\]", out)
    assert runpath, out
    parts = runpath.group(1).split(":")
    assert "$ORIGIN/../../gradient_compression_quantize_amd" in parts
    assert "$ORIGIN/../../oracle" in parts
