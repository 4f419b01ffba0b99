"""No kernel writes outside the caller's buffers.

Every output (and in-place residual) is a view one element into a larger
buffer filled with a sentinel, so that it is 4 but not 16 bytes aligned and
has guard elements on both sides. The calls run at ragged sizes (partial
tiles), through the C ABI; afterwards the results match the oracle and every
guard element still holds the sentinel.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from conftest import announce

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")

GUARD = 8          # guard elements after the view
SENT_F = -12345.0  # sentinel for float buffers
SENT_I = -777      # sentinel for int32 buffers


def guarded(n, dtype, sentinel):
    buf = torch.full((n + 1 + GUARD,), sentinel, dtype=dtype, device=gu.DEV)
    return buf, buf[1:1 + n]


def guards_intact(buf, n, sentinel):
    host = gu.host(buf)
    return host[0] == sentinel and np.all(host[1 + n:] == sentinel)


@pytest.mark.parametrize("n", [1, 17, 1023, 1025, 4099, 65_536 + 5])
def test_threshold_paths_stay_in_bounds(gcq, n):
    announce(f"guards: 2-bit and ternary n={n}")
    g = si.normal_f32(si.grad_seed(3, n % 97), n, 0.05)
    r0 = si.normal_f32(si.grad_seed(4, n % 89), n, 0.02)
    for words, comp, dsum, o_quant, o_sum in (
            (gcq.gc_compressed_2bit_words, gcq.compress_2bit, gcq.decompress_2bit_sum,
             oracle.quantize_2bit, oracle.dequantize_2bit_sum),
            (gcq.gc_compressed_ternary_words, gcq.compress_ternary, gcq.decompress_ternary_sum,
             oracle.quantize_ternary, oracle.dequantize_ternary_sum)):
        gbuf, gv = guarded(n, torch.float32, SENT_F)
        gv.copy_(torch.from_numpy(g))
        rbuf, rv = guarded(n, torch.float32, SENT_F)
        rv.copy_(torch.from_numpy(r0))
        cbuf = torch.full((words(n) + GUARD,), SENT_I, dtype=torch.int32, device=gu.DEV)
        comp(gv, rv, -0.05, 0.05, cbuf[:words(n)])
        obuf, ov = guarded(n, torch.float32, SENT_F)
        dsum([cbuf[:words(n)]] * 3, n, ov)
        gu.sync()
        r_or = r0.copy()
        c_or = o_quant(g, r_or, -0.05, 0.05)
        np.testing.assert_array_equal(gu.host(cbuf[:words(n)], np.uint32), c_or)
        assert np.all(gu.host(cbuf[words(n):]) == SENT_I), "block guard"
        np.testing.assert_array_equal(gu.host(rv).view(np.uint32), r_or.view(np.uint32))
        assert guards_intact(rbuf, n, SENT_F), "residual guard"
        assert guards_intact(gbuf, n, SENT_F), "gradient guard"
        np.testing.assert_array_equal(gu.host(ov), o_sum([c_or] * 3, n))
        assert guards_intact(obuf, n, SENT_F), "output guard"


@pytest.mark.parametrize("n", [3, 1023, 1025, 4099, 65_536 + 5])
def test_qsgd_paths_stay_in_bounds(gcq, n):
    W, s, seed = 3, 127, 23
    announce(f"guards: QSGD-MN n={n}")
    grads = [si.heavy_tailed_f32(si.grad_seed(w, 17), n, 0.02) for w in range(W)]
    gv = []
    for g in grads:
        _, v = guarded(n, torch.float32, SENT_F)
        v.copy_(torch.from_numpy(g))
        gv.append(v)
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(gv, norm, ws)
    lbufs = [torch.full((n + 4 + 4 * GUARD,), 99, dtype=torch.int8, device=gu.DEV)
             for _ in range(W)]
    levels = [b[4:4 + n] for b in lbufs]  # 4-byte offset: the word paths
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(gv[w], norm, s, seed, w, levels[w])
    sbuf, sv = guarded(n, torch.int32, SENT_I)
    obuf, ov = guarded(n, torch.float32, SENT_F)
    gcq.qsgd_dequant_sum(levels, norm, s, ov, sums=sv)
    fsbuf, fsv = guarded(n, torch.int32, SENT_I)
    fobuf, fov = guarded(n, torch.float32, SENT_F)
    gcq.qsgd_quantize_sum(gv, norm, s, seed, fov, sums=fsv)
    gu.sync()
    nrm = oracle.maxnorm(grads)
    assert np.float32(gu.host(norm)[0]) == nrm
    lv_or = [oracle.qsgd_quantize(g, nrm, s, seed, w) for w, g in enumerate(grads)]
    for w in range(W):
        np.testing.assert_array_equal(gu.host(levels[w]), lv_or[w])
        host = gu.host(lbufs[w])
        assert np.all(host[:4] == 99) and np.all(host[4 + n:] == 99), "levels guard"
    S = oracle.level_sum(lv_or)
    d = oracle.qsgd_dequantize(S, nrm, s)
    for sb, svw, ob, ovw, what in ((sbuf, sv, obuf, ov, "level sum"),
                                   (fsbuf, fsv, fobuf, fov, "fused")):
        np.testing.assert_array_equal(gu.host(svw), S, err_msg=what)
        np.testing.assert_array_equal(gu.host(ovw), d, err_msg=what)
        assert guards_intact(sb, n, SENT_I), f"{what}: sums guard"
        assert guards_intact(ob, n, SENT_F), f"{what}: output guard"
