"""Hot-path steps captured once as HIP graphs and replayed, through the C ABI.

Each step is captured after a warm-up call on the capture stream (which
counts as its first iteration), then replayed four times. Before every
replay the test writes the next iteration's gradients into the captured
buffers and poisons the outputs with eager device work, and synchronizes.
Each replay must match the oracle's run of that iteration bit for bit (the
dequantized sums are bit-exact too; their 1e-6 relative bar is checked as
well). Error-feedback residuals carry from replay to replay, as they do
between training steps.

Steps: the 2-bit error-feedback step (W compresses + the W-block
dequantize-and-sum), the same with ternary packing, the many-tensor compress,
and the QSGD-MN step (max-norm, W quantizes, level sum and dequantize, and the
fused quantize-sum beside it).
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

REPLAYS = 4


def capture(step):
    """Warm-up call on a side stream (capture needs one), then the capture."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    gu.sync()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    gu.sync()
    return graph


def load(dst, arrays):
    for d, a in zip(dst, arrays):
        d.copy_(torch.from_numpy(a))


def check_sum(got, expect):
    assert np.all(np.abs(got.astype(np.float64) - expect) <= 1e-6 * np.abs(expect.astype(np.float64)))
    np.testing.assert_array_equal(got.view(np.uint32), expect.view(np.uint32))


@pytest.mark.parametrize("packing", ["2bit", "ternary"])
def test_threshold_ef_step_in_hip_graph(gcq, packing):
    n, W, thr = 100_003, 4, 0.05
    announce(f"{packing} EF step captured in a HIP graph, {REPLAYS} replays")
    if packing == "2bit":
        words = gcq.gc_compressed_2bit_words(n)
        compress, dsum = gcq.compress_2bit, gcq.decompress_2bit_sum
        o_quant, o_sum = oracle.quantize_2bit, oracle.dequantize_2bit_sum
    else:
        words = gcq.gc_compressed_ternary_words(n)
        compress, dsum = gcq.compress_ternary, gcq.decompress_ternary_sum
        o_quant, o_sum = oracle.quantize_ternary, oracle.dequantize_ternary_sum
    g_dev = [gu.empty(n, torch.float32) for _ in range(W)]
    r_dev = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for _ in range(W)]
    c_dev = [gu.empty(words, torch.int32) for _ in range(W)]
    out = gu.empty(n, torch.float32)
    r_or = [np.zeros(n, np.float32) for _ in range(W)]

    def grads_of(t):
        return [si.normal_f32(si.grad_seed(w, 40 + t), n, 0.05) for w in range(W)]

    def step():
        for w in range(W):
            compress(g_dev[w], r_dev[w], -thr, thr, c_dev[w])
        dsum(c_dev, n, out)

    def check(t, grads):
        c_or = [o_quant(grads[w], r_or[w], -thr, thr) for w in range(W)]
        for w in range(W):
            np.testing.assert_array_equal(gu.host(c_dev[w], np.uint32), c_or[w],
                                          err_msg=f"iteration {t} worker {w}")
            np.testing.assert_array_equal(gu.host(r_dev[w]).view(np.uint32),
                                          r_or[w].view(np.uint32))
        check_sum(gu.host(out), o_sum(c_or, n))

    grads = grads_of(0)
    load(g_dev, grads)
    gu.sync()
    graph = capture(step)  # its warm-up ran iteration 0
    check(0, grads)
    for t in range(1, 1 + REPLAYS):
        grads = grads_of(t)
        load(g_dev, grads)
        for c in c_dev:
            c.fill_(-1)
        out.fill_(float("nan"))
        gu.sync()
        graph.replay()
        gu.sync()
        check(t, grads)


def test_multi_tensor_compress_in_hip_graph(gcq):
    sizes = [768, 3, 100_003, 0, 30_000, 4096]
    neg, pos = -0.005, 0.005
    announce(f"many-tensor compress captured in a HIP graph, {REPLAYS} replays")
    g_dev = [gu.empty(k, torch.float32) for k in sizes]
    r_dev = [torch.zeros(k, dtype=torch.float32, device=gu.DEV) for k in sizes]
    r_or = [np.zeros(k, np.float32) for k in sizes]
    plan = gcq.Plan2bitMulti(g_dev, r_dev)
    offs = plan.block_offsets()
    compr = gu.empty(plan.compressed_words, torch.int32)

    def grads_of(t):
        return [si.normal_f32(900 + 10 * i + t, k, 0.005) for i, k in enumerate(sizes)]

    def check(t, grads):
        got = gu.host(compr, np.uint32)
        for i, k in enumerate(sizes):
            c_or = oracle.quantize_2bit(grads[i], r_or[i], neg, pos)
            np.testing.assert_array_equal(got[offs[i]:offs[i] + c_or.size], c_or,
                                          err_msg=f"iteration {t} tensor {i}")
            np.testing.assert_array_equal(gu.host(r_dev[i]).view(np.uint32),
                                          r_or[i].view(np.uint32))

    try:
        grads = grads_of(0)
        load(g_dev, grads)
        gu.sync()
        graph = capture(lambda: plan.compress(neg, pos, compr))
        check(0, grads)
        for t in range(1, 1 + REPLAYS):
            grads = grads_of(t)
            load(g_dev, grads)
            compr.fill_(-1)
            gu.sync()
            graph.replay()
            gu.sync()
            check(t, grads)
    finally:
        plan.destroy()


def test_qsgd_step_in_hip_graph(gcq):
    n, W, s, seed = 100_003, 4, 127, 77
    announce(f"QSGD-MN step (plain and fused) captured in a HIP graph, {REPLAYS} replays")
    g_dev = [gu.empty(n, torch.float32) for _ in range(W)]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    levels = [gu.empty(n, torch.int8) for _ in range(W)]
    sums = gu.empty(n, torch.int32)
    out = gu.empty(n, torch.float32)
    fsums = gu.empty(n, torch.int32)
    fout = gu.empty(n, torch.float32)

    def grads_of(t):
        return [si.heavy_tailed_f32(si.grad_seed(w, 60 + t), n, 0.02) for w in range(W)]

    def step():
        gcq.qsgd_global_maxnorm(g_dev, norm, ws)
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, levels[w])
        gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)
        gcq.qsgd_quantize_sum(g_dev, norm, s, seed, fout, sums=fsums)

    def check(t, grads):
        nrm = oracle.maxnorm(grads)
        assert gu.host(norm)[0] == nrm, f"iteration {t} norm"
        lv = [oracle.qsgd_quantize(g, nrm, s, seed, w) for w, g in enumerate(grads)]
        for w in range(W):
            np.testing.assert_array_equal(gu.host(levels[w]), lv[w],
                                          err_msg=f"iteration {t} worker {w}")
        S = oracle.level_sum(lv)
        d = oracle.qsgd_dequantize(S, nrm, s)
        np.testing.assert_array_equal(gu.host(sums), S)
        np.testing.assert_array_equal(gu.host(fsums), S)
        check_sum(gu.host(out), d)
        check_sum(gu.host(fout), d)

    grads = grads_of(0)
    load(g_dev, grads)
    gu.sync()
    graph = capture(step)
    check(0, grads)
    for t in range(1, 1 + REPLAYS):
        grads = grads_of(t)
        load(g_dev, grads)
        norm.fill_(float("nan"))
        for lv in levels:
            lv.fill_(-128)
        for buf in (sums, fsums):
            buf.fill_(-1)
        for buf in (out, fout):
            buf.fill_(float("nan"))
        gu.sync()
        graph.replay()
        gu.sync()
        check(t, grads)


def test_capture_before_any_eager_call(gcq):
    """The launch paths' one-time queries (each capped kernel's own LDS, the
    device's LDS size) first run inside a graph capture, in a fresh child
    process (capture_first_check.py): the capture succeeds and its replays
    match the oracle."""
    import os
    import subprocess
    import sys
    announce("graph captured before any eager library call (child process)")
    script = os.path.join(os.path.dirname(__file__), "capture_first_check.py")
    res = subprocess.run([sys.executable, "-u", script], capture_output=True, text=True,
                         timeout=110)
    print(res.stdout[-2000:], res.stderr[-2000:])
    assert res.returncode == 0 and res.stdout.strip().endswith("OK")
