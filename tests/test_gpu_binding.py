"""The binding's launch target on a GPU: the device and stream it hands the
library are torch's current ones (read from torch's C layer when it offers
them), under a side stream too, and a call on a side stream produces the
same result as one on the default stream."""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def handle(stream_arg, gcq) -> int:
    """The stream handle the binding passes (the null stream reads as 0)."""
    return gcq._stream(stream_arg).value or 0


def test_current_device_and_stream_match_torch(gcq):
    announce("binding: current device and stream")
    assert gcq._current_device() == torch.cuda.current_device()
    assert handle(None, gcq) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert handle(None, gcq) == side.cuda_stream != 0
    assert handle(None, gcq) == torch.cuda.current_stream().cuda_stream
    assert handle(side, gcq) == side.cuda_stream


def test_compress_on_a_side_stream_matches_the_oracle(gcq):
    """compress_2bit issued with no stream argument inside a side-stream
    context runs on that stream: its result, synchronised through that
    stream only, equals the oracle's."""
    announce("binding: compress_2bit on a side stream")
    n = 100_003
    g = si.normal_f32(si.grad_seed(0, 11), n, 0.5)
    r0 = si.normal_f32(si.grad_seed(1, 11), n, 0.2)
    res_or = r0.copy()
    words_or = oracle.quantize_2bit(g, res_or, -0.5, 0.5)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g_dev, r_dev = gu.dev(g), gu.dev(r0)
    out = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        gcq.compress_2bit(g_dev, r_dev, -0.5, 0.5, out)
    side.synchronize()
    np.testing.assert_array_equal(gu.host(out, np.uint32), words_or)
    np.testing.assert_array_equal(gu.host(r_dev).view(np.uint32), res_or.view(np.uint32))
