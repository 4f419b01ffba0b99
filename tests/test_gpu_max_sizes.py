"""Parity at sizes past the 32-bit boundaries of the index arithmetic,
checked against the oracle on windows and samples, and by properties over
every element (the oracle cannot take tens of GB in reasonable time):

* 2-bit and ternary blocks of n = 2^32 + 1029 values: value indices above
  2^32, word indices above 2^28;
* QSGD-MN over n = 2^34 + 4109 values: slot indices above 2^32, so the
  Philox counter's high word is nonzero for the last slots;
* the one-call GlobalRandK-MN step at n = 2^32, the largest size the draw
  accepts.

Inputs: uniform [-1, 1) fp32 drawn on the device by a seeded generator
(synthetic_inputs.uniform_f32_device), windows copied back for the oracle.
Each test needs tens of GB of device memory and skips, saying so, when the
device has less free; each frees what it allocated.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

gu = pytest.importorskip("gpu_util")

GiB = 1 << 30


def need(bytes_):
    torch.cuda.synchronize()
    torch.cuda.empty_cache()  # memory earlier tests left in torch's cache
    free, _ = torch.cuda.mem_get_info()
    if free < bytes_ + 4 * GiB:
        pytest.skip(f"needs {bytes_ / GiB:.0f} GiB of free device memory, {free / GiB:.0f} GiB free")


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_2bit_and_ternary_beyond_2e32_values(gcq):
    n = (1 << 32) + 1029
    need(4 * n * 4 + 2 * GiB)
    announce(f"max size: 2-bit and ternary, n={n}")
    g = si.uniform_f32_device(41, n)
    g.mul_(0.5)
    r2 = si.uniform_f32_device(42, n)
    r2.mul_(0.25)
    r3 = r2.clone()
    c2 = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1)
    c3 = gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32, fill=-1)
    # windows of whole words of both packings (starts and lengths multiples
    # of 80 = lcm(16, 20)), the last one running to n
    def at(v):
        return v - v % 80
    wins = [(0, 8000), (at((1 << 31) - 4000), at((1 << 31) - 4000) + 8000),
            (at((1 << 32) - 4000), n)]
    r_before = [r2[lo:hi].cpu().numpy() for lo, hi in wins]
    g_win = [g[lo:hi].cpu().numpy() for lo, hi in wins]
    gcq.compress_2bit(g, r2, -0.3, 0.3, c2)
    gcq.compress_ternary(g, r3, -0.3, 0.3, c3)
    out = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.decompress_2bit(c2, n, out)
    gu.sync()
    h2 = c2[:3].cpu().numpy().view(np.uint32)
    h3 = c3[:3].cpu().numpy().view(np.uint32)
    hdr = oracle.quantize_2bit(np.zeros(0, np.float32), np.zeros(0, np.float32), -0.3, 0.3)
    assert h2[0] == hdr[0] and h2[1] == hdr[1] and h3[0] == hdr[0] and h3[1] == hdr[1]
    assert h2[2] == np.float32(n).view(np.uint32) == h3[2]
    for (lo, hi), gw, rw in zip(wins, g_win, r_before):
        announce(f"max size: window [{lo}, {hi})")
        r_or2, r_or3 = rw.copy(), rw.copy()
        w2 = oracle.quantize_2bit(gw, r_or2, -0.3, 0.3)[3:]
        w3 = oracle.quantize_ternary(gw, r_or3, -0.3, 0.3)[3:]
        np.testing.assert_array_equal(c2[3 + lo // 16:3 + lo // 16 + w2.size].cpu().numpy().view(np.uint32), w2)
        np.testing.assert_array_equal(c3[3 + lo // 20:3 + lo // 20 + w3.size].cpu().numpy().view(np.uint32), w3)
        np.testing.assert_array_equal(r2[lo:hi].cpu().numpy().view(np.uint32), r_or2.view(np.uint32))
        np.testing.assert_array_equal(r3[lo:hi].cpu().numpy().view(np.uint32), r_or3.view(np.uint32))
        np.testing.assert_array_equal(out[lo:hi].cpu().numpy(),
                                      oracle.dequantize_2bit(oracle.quantize_2bit(gw, rw.copy(), -0.3, 0.3), hi - lo))
    # every element: the two packings left the same residuals
    assert torch.equal(r2.view(torch.int32), r3.view(torch.int32))
    del g, r2, r3, c2, c3, out
    release()


def test_2bit_misaligned_beyond_2e32_values(gcq):
    """The lane-contiguous 4-byte paths (gradient, residual and output 4 bytes
    off 16-byte alignment) past the 32-bit index boundaries."""
    n = (1 << 32) + 1029
    need(3 * (n + 1) * 4 + 2 * GiB)
    announce(f"max size: 2-bit, buffers 4 bytes off alignment, n={n}")
    g_buf = si.uniform_f32_device(43, n + 1)
    g_buf.mul_(0.5)
    r_buf = si.uniform_f32_device(44, n + 1)
    r_buf.mul_(0.25)
    g, r = g_buf[1:], r_buf[1:]
    assert g.data_ptr() % 16 != 0 and r.data_ptr() % 16 != 0
    c2 = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1)
    wins = [(0, 8000), ((1 << 31) - 4000, (1 << 31) + 4000), ((1 << 32) - 4000, n)]
    r_before = [r[lo:hi].cpu().numpy() for lo, hi in wins]
    g_win = [g[lo:hi].cpu().numpy() for lo, hi in wins]
    gcq.compress_2bit(g, r, -0.3, 0.3, c2)
    del g_buf, g
    out_buf = gu.empty(n + 1, torch.float32, fill=float("nan"))
    out = out_buf[1:]
    gcq.decompress_2bit(c2, n, out)
    gu.sync()
    for (lo, hi), gw, rw in zip(wins, g_win, r_before):
        announce(f"max size misaligned: window [{lo}, {hi})")
        r_or = rw.copy()
        w2 = oracle.quantize_2bit(gw, r_or, -0.3, 0.3)[3:]
        np.testing.assert_array_equal(c2[3 + lo // 16:3 + lo // 16 + w2.size].cpu().numpy().view(np.uint32), w2)
        np.testing.assert_array_equal(r[lo:hi].cpu().numpy().view(np.uint32), r_or.view(np.uint32))
        np.testing.assert_array_equal(out[lo:hi].cpu().numpy(),
                                      oracle.dequantize_2bit(oracle.quantize_2bit(gw, rw.copy(), -0.3, 0.3), hi - lo))
    del r_buf, r, c2, out_buf, out
    release()


def test_qsgd_beyond_2e32_slots(gcq):
    n = (1 << 34) + 4109
    need(n * 4 + n + 2 * GiB)
    announce(f"max size: QSGD-MN, n={n}")
    s, seed = 127, 77
    g = si.uniform_f32_device(43, n)
    j = (1 << 34) + 17
    g[j] = -1.5  # the max |g|, in the last slots
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(1, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm([g], norm, ws)
    lv = gu.empty(n, torch.int8, fill=99)
    gcq.qsgd_maxnorm_quantize(g, norm, s, seed, 0, lv)
    gu.sync()
    assert float(norm.item()) == 1.5
    rng = np.random.default_rng(5)
    samp = np.unique(np.concatenate([rng.integers(0, n, 200_000, dtype=np.int64),
                                     np.arange(0, 64), np.arange((1 << 34) - 4096, n),
                                     np.arange((1 << 33) - 64, (1 << 33) + 64)]))
    samp_t = torch.from_numpy(samp).to(gu.DEV)
    vals = g[samp_t].cpu().numpy()
    got = lv[samp_t].cpu().numpy()
    np.testing.assert_array_equal(got, oracle.qsgd_quantize_at(vals, samp.astype(np.uint64),
                                                              np.float32(1.5), s, seed, 0))
    assert int(lv[j].item()) == -s
    assert int(lv.abs().max().item()) <= s
    del lv
    release()
    # the fused form (W = 1, no sums) over the same gradient
    free, _ = torch.cuda.mem_get_info()
    if free >= n * 4 + 4 * GiB:
        announce("max size: fused quantize-sum")
        out = gu.empty(n, torch.float32)
        gcq.qsgd_quantize_sum([g], norm, s, seed, out)
        gu.sync()
        lv_or = oracle.qsgd_quantize_at(vals, samp.astype(np.uint64), np.float32(1.5), s, seed, 0)
        np.testing.assert_array_equal(out[samp_t].cpu().numpy(),
                                      oracle.qsgd_dequantize(lv_or.astype(np.int32), np.float32(1.5), s))
        del out
    del g
    release()


def test_grandk_mn_step_at_n_2e32(gcq):
    n, K, W, s, seed = 1 << 32, 10_000, 2, 7, 3
    need(3 * n * 4 + GiB)
    announce(f"max size: grandk_mn_step n={n} K={K} W={W}")
    grads = [si.uniform_f32_device(44 + w, n) for w in range(W)]
    idx = gu.empty(K, torch.int32)
    sums = gu.empty(K, torch.int32)
    dense = gu.empty(n, torch.float32, fill=float("nan"))
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_mn_step(grads, K, seed, s, idx, dense, ws, sums=sums)
    gu.sync()
    announce("max size: oracle draw over 2^32 positions")
    idx_or = oracle.randk_indices(n, K, seed)
    np.testing.assert_array_equal(gu.host(idx, np.uint32), idx_or)
    it = torch.from_numpy(idx_or.astype(np.int64)).to(gu.DEV)
    gk = [g[it].cpu().numpy() for g in grads]
    nk = oracle.maxnorm(gk)
    S = oracle.level_sum([oracle.qsgd_quantize(x, nk, s, seed, w) for w, x in enumerate(gk)])
    np.testing.assert_array_equal(gu.host(sums), S)
    vals = oracle.qsgd_dequantize(S, nk, s)
    np.testing.assert_array_equal(dense[it].cpu().numpy(), vals)
    # everywhere else zero: the nonzeros of the dense output are exactly the
    # nonzero values at the drawn indices
    assert int(torch.count_nonzero(dense).item()) == int(np.count_nonzero(vals))
    assert not bool(torch.isnan(dense).any().item())
    del grads, dense, ws
    release()
