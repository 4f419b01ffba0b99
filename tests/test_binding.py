"""The Python binding's own checks, without a GPU: it rejects host tensors,
wrong dtypes, non-contiguous tensors and undersized buffers before calling
the library, and turns the library's host-side validation failures into
GcqError. A stub stands in for a device tensor where one is needed; nothing
here launches a kernel.
"""
import pytest
import torch

import gradient_compression_quantize_amd as gcq


class FakeDev:
    """Looks like a contiguous device tensor to the binding; its address is
    never dereferenced (the calls below fail validation first)."""

    def __init__(self, n, dtype=torch.float32, contiguous=True, addr=0x10000):
        self._n, self.dtype, self._c, self._a = n, dtype, contiguous, addr
        self.is_cuda = True
        self.device_index = 0

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return self._c

    def data_ptr(self):
        return self._a

    def get_device(self):
        return self.device_index


class FakeStream:
    cuda_stream = 0


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not gcq.LIB_PATH.exists():
        pytest.fail("libgcq.so is not built (python gradient_compression_quantize_amd/build.py)")
    gcq.load()


def test_host_tensors_are_rejected():
    g, r = torch.zeros(32), torch.zeros(32)
    c = torch.zeros(gcq.gc_compressed_2bit_words(32), dtype=torch.int32)
    with pytest.raises(TypeError, match="device tensor"):
        gcq.compress_2bit(g, r, -1.0, 1.0, c)
    with pytest.raises(TypeError, match="device tensor"):
        gcq.compress_ternary(g, r, -1.0, 1.0, torch.zeros(5, dtype=torch.int32))


def test_dtype_and_layout_are_checked():
    n = 64
    words = gcq.gc_compressed_2bit_words(n)
    with pytest.raises(TypeError, match="float32"):
        gcq.compress_2bit(FakeDev(n, torch.float16), FakeDev(n), -1.0, 1.0,
                          FakeDev(words, torch.int32), stream=FakeStream())
    with pytest.raises(TypeError, match="int32"):
        gcq.compress_2bit(FakeDev(n), FakeDev(n), -1.0, 1.0, FakeDev(words, torch.float32),
                          stream=FakeStream())
    with pytest.raises(TypeError, match="contiguous"):
        gcq.decompress_2bit(FakeDev(words, torch.int32), n, FakeDev(n, contiguous=False),
                            stream=FakeStream())


def test_tensors_and_streams_on_another_device_are_rejected(monkeypatch):
    """The library launches on the current device: a tensor or an explicit
    stream on another one is refused before any call (torch's device queries
    are stubbed so that the check runs without a GPU)."""
    monkeypatch.setattr(gcq, "_gpu_present", True)
    monkeypatch.setattr(torch.cuda, "current_device", lambda: 0)
    n = 64
    words = gcq.gc_compressed_2bit_words(n)
    other = FakeDev(n)
    other.device_index = 1
    with pytest.raises(ValueError, match="residual: on cuda:1 but the current device is cuda:0"):
        gcq.compress_2bit(FakeDev(n), other, -1.0, 1.0, FakeDev(words, torch.int32),
                          stream=FakeStream())

    class OtherStream(FakeStream):
        device = torch.device("cuda", 1)

    with pytest.raises(ValueError, match="stream is on cuda:1"):
        gcq.compress_2bit(FakeDev(n), FakeDev(n), -1.0, 1.0, FakeDev(words, torch.int32),
                          stream=OtherStream())


def test_undersized_buffers_are_rejected():
    n = 1000
    with pytest.raises(ValueError, match="differ in size"):
        gcq.compress_2bit(FakeDev(n), FakeDev(n - 1), -1.0, 1.0,
                          FakeDev(gcq.gc_compressed_2bit_words(n), torch.int32))
    with pytest.raises(ValueError, match="too small"):
        gcq.compress_2bit(FakeDev(n), FakeDev(n), -1.0, 1.0,
                          FakeDev(gcq.gc_compressed_2bit_words(n) - 1, torch.int32))
    with pytest.raises(ValueError, match="too small"):
        gcq.compress_ternary(FakeDev(n), FakeDev(n), -1.0, 1.0,
                             FakeDev(gcq.gc_compressed_ternary_words(n) - 1, torch.int32))
    with pytest.raises(ValueError, match="too small"):
        gcq.decompress_2bit(FakeDev(gcq.gc_compressed_2bit_words(n), torch.int32), n,
                            FakeDev(n - 1))
    with pytest.raises(ValueError, match="too small"):
        gcq.decompress_ternary_sum([FakeDev(gcq.gc_compressed_ternary_words(n) - 1, torch.int32)],
                                   n, FakeDev(n))
    with pytest.raises(ValueError, match="differ in size"):
        gcq.qsgd_quantize_sum([FakeDev(n), FakeDev(n + 1)], FakeDev(1), 7, 0, FakeDev(n))
    with pytest.raises(ValueError, match="too small"):
        gcq.grandk_mn_step([FakeDev(n)], 100, 0, 7, FakeDev(99, torch.int32), FakeDev(n),
                           FakeDev(1 << 20, torch.uint8))


def test_scatter_sums_and_norm_sizes_are_checked():
    """The scatter form writes sums[k] for every k < n, and every QSGD call
    reads (or writes) norm[0]: short buffers are refused before the call."""
    n, dense_n = 100, 1000
    lv = [FakeDev(n, torch.int8), FakeDev(n, torch.int8)]
    with pytest.raises(ValueError, match="sums too small"):
        gcq.qsgd_dequant_sum(lv, FakeDev(1), 7, FakeDev(dense_n), sums=FakeDev(n - 1, torch.int32),
                             scatter_idx=FakeDev(n, torch.int32), dense_n=dense_n)
    empty_norm = FakeDev(0)
    with pytest.raises(ValueError, match="norm must hold"):
        gcq.qsgd_dequant_sum(lv, empty_norm, 7, FakeDev(n))
    with pytest.raises(ValueError, match="norm must hold"):
        gcq.qsgd_global_maxnorm([FakeDev(n)], empty_norm, FakeDev(1 << 16, torch.uint8))
    with pytest.raises(ValueError, match="norm must hold"):
        gcq.qsgd_maxnorm_quantize(FakeDev(n), empty_norm, 7, 0, 0, FakeDev(n, torch.int8))
    with pytest.raises(ValueError, match="norm must hold"):
        gcq.qsgd_quantize_sum([FakeDev(n)], empty_norm, 7, 0, FakeDev(n))
    with pytest.raises(ValueError, match="norm must hold"):
        gcq.grandk_mn_step([FakeDev(n)], 10, 0, 7, FakeDev(10, torch.int32), FakeDev(n),
                           FakeDev(1 << 20, torch.uint8), norm=empty_norm)


def test_library_validation_surfaces_as_gcq_error():
    n = 64
    words = gcq.gc_compressed_2bit_words(n)
    with pytest.raises(gcq.GcqError, match="threshold") as e:
        gcq.compress_2bit(FakeDev(n), FakeDev(n), 0.5, 1.0, FakeDev(words, torch.int32),
                          stream=FakeStream())
    assert e.value.code == gcq.GC_EINVAL
    with pytest.raises(gcq.GcqError, match="s must be") as e:
        gcq.qsgd_quantize_sum([FakeDev(n)], FakeDev(1), 0, 0, FakeDev(n), stream=FakeStream())
    assert e.value.code == gcq.GC_EINVAL
    with pytest.raises(gcq.GcqError, match="K <= n"):
        gcq.grandk_mn_step([FakeDev(n)], n + 1, 0, 7, FakeDev(n + 1, torch.int32), FakeDev(n),
                           FakeDev(1 << 20, torch.uint8), stream=FakeStream())
    with pytest.raises(gcq.GcqError, match="workspace too small"):
        gcq.grandk_mn_step([FakeDev(n)], 10, 0, 7, FakeDev(10, torch.int32), FakeDev(n),
                           FakeDev(16, torch.uint8), stream=FakeStream())


def test_workspace_queries_need_no_gpu():
    assert gcq.qsgd_maxnorm_ws_bytes(8, 138_357_544) == 8 * 4095 * 4
    assert gcq.grandk_ws_bytes(25_557_032, 10_000) == 4 * (32768 + 2 * 10_000)
    assert gcq.grandk_mn_step_ws_bytes(8, 25_557_032, 10_000) >= 8 * 10_000 * 4
