"""Parity of the striding kernel paths, run in a child process whose
GCQ_MAX_GRID_BLOCKS caps every launch at a few workgroups (the library reads
the variable once, when it is first used). Exits 0 when every result matches
the oracle; prints the failing case otherwise.
"""
import os
import pathlib
import sys

ROOT = pathlib.Path(__file__).resolve().parent.parent
sys.path.insert(0, str(ROOT))
sys.path.insert(0, str(ROOT / "tests"))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import gradient_compression_quantize_amd as gcq  # noqa: E402
import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402
import gpu_util as gu  # noqa: E402


def check(cond, what):
    if not cond:
        print(f"FAIL: {what}", flush=True)
        sys.exit(1)


def main():
    assert os.environ.get("GCQ_MAX_GRID_BLOCKS"), "run with GCQ_MAX_GRID_BLOCKS set"
    gcq.load()
    # 2-bit: vector path over many more tiles than waves, ragged tail; and
    # the same with buffers 4 bytes off 16-byte alignment (lane-contiguous
    # 4-byte accesses)
    for n, mis in ((40_000 + 5, False), (123_457, False), (40_000 + 5, True), (123_457, True)):
        print(f"[case] capped compress/decompress n={n} misaligned={mis}", flush=True)
        g = si.normal_f32(n, n, 0.5)
        r0 = si.normal_f32(n + 1, n, 0.2)
        r_dev = gu.dev(r0, mis)
        compr = gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32, fill=-1)
        gcq.compress_2bit(gu.dev(g, mis), r_dev, -0.5, 0.5, compr)
        r_or = r0.copy()
        c_or = oracle.quantize_2bit(g, r_or, -0.5, 0.5)
        gu.sync()
        check(np.array_equal(gu.host(compr, np.uint32), c_or), f"compress words n={n}")
        check(np.array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32)),
              f"compress residual n={n}")
        base = si.normal_f32(n + 2, n, 1.0)
        out = gu.dev(base, mis)
        gcq.decompress_2bit(gu.dev(c_or), n, out, accumulate=True)
        gu.sync()
        check(np.array_equal(gu.host(out), (base + oracle.dequantize_2bit(c_or, n)).astype(np.float32)),
              f"decompress accumulate n={n}")
        for W in (8, 9):
            comprs = [oracle.quantize_2bit(si.normal_f32(7 * w + n, n, 0.5), np.zeros(n, np.float32),
                                           -0.3 - 0.01 * w, 0.3 + 0.01 * w) for w in range(W)]
            out = gu.empty(n, torch.float32, misalign=mis, fill=float("nan"))
            gcq.decompress_2bit_sum([gu.dev(c) for c in comprs], n, out)
            gu.sync()
            check(np.array_equal(gu.host(out), oracle.dequantize_2bit_sum(comprs, n)),
                  f"decompress sum W={W} n={n}")
    # ternary packing: same shapes, aligned and 4 bytes off alignment
    for n, mis in ((40_000 + 7, False), (123_457, False), (40_000 + 7, True), (123_457, True)):
        print(f"[case] capped ternary n={n} misaligned={mis}", flush=True)
        g = si.normal_f32(n + 3, n, 0.5)
        r0 = si.normal_f32(n + 4, n, 0.2)
        r_dev = gu.dev(r0, mis)
        compr = gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32, fill=-1)
        gcq.compress_ternary(gu.dev(g, mis), r_dev, -0.5, 0.5, compr)
        r_or = r0.copy()
        c_or = oracle.quantize_ternary(g, r_or, -0.5, 0.5)
        gu.sync()
        check(np.array_equal(gu.host(compr, np.uint32), c_or), f"ternary words n={n}")
        check(np.array_equal(gu.host(r_dev).view(np.uint32), r_or.view(np.uint32)),
              f"ternary residual n={n}")
        base = si.normal_f32(n + 5, n, 1.0)
        out = gu.dev(base, mis)
        gcq.decompress_ternary(gu.dev(c_or), n, out, accumulate=True)
        gu.sync()
        check(np.array_equal(gu.host(out), (base + oracle.dequantize_ternary(c_or, n)).astype(np.float32)),
              f"ternary decompress accumulate n={n}")
        for W in (8, 9):
            comprs = [oracle.quantize_ternary(si.normal_f32(11 * w + n, n, 0.5), np.zeros(n, np.float32),
                                              -0.3 - 0.01 * w, 0.3 + 0.02 * w) for w in range(W)]
            out = gu.empty(n, torch.float32, misalign=mis, fill=float("nan"))
            gcq.decompress_ternary_sum([gu.dev(c) for c in comprs], n, out)
            gu.sync()
            check(np.array_equal(gu.host(out), oracle.dequantize_ternary_sum(comprs, n)),
                  f"ternary decompress sum W={W} n={n}")
    # many tensors, more chunks than workgroups
    print("[case] capped multi-tensor", flush=True)
    sizes = [5000, 0, 17, 70_001, 4096 * 3, 33]
    grads = [gu.empty(n, torch.float32) for n in sizes]
    res = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for n in sizes]
    plan = gcq.Plan2bitMulti(grads, res)
    blocks = []
    for t, n in enumerate(sizes):
        g = si.normal_f32(300 + t, n, 0.5)
        grads[t].copy_(torch.from_numpy(g))
        blocks.append(oracle.quantize_2bit(g, np.zeros(n, np.float32), -0.5, 0.5))
    compr = gu.empty(plan.compressed_words, torch.int32, fill=-1)
    plan.compress(-0.5, 0.5, compr)
    gu.sync()
    check(np.array_equal(gu.host(compr, np.uint32), np.concatenate(blocks)), "multi-tensor blocks")
    plan.destroy()
    # QSGD step and GRandK gather with a capped grid
    print("[case] capped qsgd", flush=True)
    n, W, s, seed = 50_003, 3, 127, 11
    gs = [si.heavy_tailed_f32(400 + w, n, 0.02) for w in range(W)]
    g_dev = [gu.dev(g) for g in gs]
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    gcq.qsgd_global_maxnorm(g_dev, norm, ws)
    lv = [gu.empty(n, torch.int8) for _ in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, lv[w])
    sums = gu.empty(n, torch.int32)
    out = gu.empty(n, torch.float32)
    gcq.qsgd_dequant_sum(lv, norm, s, out, sums=sums)
    gu.sync()
    norm_or = oracle.maxnorm(gs)
    lv_or = [oracle.qsgd_quantize(g, norm_or, s, seed, w) for w, g in enumerate(gs)]
    for w in range(W):
        check(np.array_equal(gu.host(lv[w]), lv_or[w]), f"qsgd levels worker {w}")
    s_or = oracle.level_sum(lv_or)
    check(np.array_equal(gu.host(sums), s_or), "qsgd sums")
    check(np.array_equal(gu.host(out), oracle.qsgd_dequantize(s_or, norm_or, s)), "qsgd dequantized")
    # the fused quantize + level sum: W read at run time (3) and known at
    # compile time (8), many more tiles than waves
    for Wf in (3, 8):
        print(f"[case] capped qsgd_quantize_sum W={Wf}", flush=True)
        gf = gs if Wf == W else [si.heavy_tailed_f32(600 + w, n, 0.02) for w in range(Wf)]
        gf_dev = [gu.dev(g) for g in gf]
        nrm_f = oracle.maxnorm(gf)
        norm_f = torch.tensor([nrm_f], dtype=torch.float32, device=gu.DEV)
        sums_f = gu.empty(n, torch.int32)
        out_f = gu.empty(n, torch.float32, fill=float("nan"))
        gcq.qsgd_quantize_sum(gf_dev, norm_f, s, seed, out_f, sums=sums_f)
        gu.sync()
        S_f = oracle.level_sum([oracle.qsgd_quantize(g, nrm_f, s, seed, w) for w, g in enumerate(gf)])
        check(np.array_equal(gu.host(sums_f), S_f), f"qsgd_quantize_sum sums W={Wf}")
        check(np.array_equal(gu.host(out_f), oracle.qsgd_dequantize(S_f, nrm_f, s)),
              f"qsgd_quantize_sum dequantized W={Wf}")
    # the same QSGD calls on buffers 4 bytes off 16-byte alignment (staged
    # loads and stores), many more tiles than waves
    print("[case] capped qsgd, misaligned buffers", flush=True)
    gm_dev = [gu.dev(g, True) for g in gs]
    gcq.qsgd_global_maxnorm(gm_dev, norm, ws)
    lvm = [gu.empty(n, torch.int8, misalign=True) for _ in range(W)]
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(gm_dev[w], norm, s, seed, w, lvm[w])
    sums_m = gu.empty(n, torch.int32, misalign=True)
    out_m = gu.empty(n, torch.float32, misalign=True, fill=float("nan"))
    gcq.qsgd_dequant_sum(lvm, norm, s, out_m, sums=sums_m)
    fsums_m = gu.empty(n, torch.int32, misalign=True)
    fout_m = gu.empty(n, torch.float32, misalign=True, fill=float("nan"))
    gcq.qsgd_quantize_sum(gm_dev, norm, s, seed, fout_m, sums=fsums_m)
    gu.sync()
    check(float(gu.host(norm)[0]) == float(norm_or), "qsgd misaligned norm")
    for w in range(W):
        check(np.array_equal(gu.host(lvm[w]), lv_or[w]), f"qsgd misaligned levels worker {w}")
    check(np.array_equal(gu.host(sums_m), s_or) and np.array_equal(gu.host(fsums_m), s_or),
          "qsgd misaligned sums")
    d_or = oracle.qsgd_dequantize(s_or, norm_or, s)
    check(np.array_equal(gu.host(out_m), d_or) and np.array_equal(gu.host(fout_m), d_or),
          "qsgd misaligned dequantized")
    # int8 levels 1-3 bytes past a 4-byte boundary (a different offset per
    # worker), gradients aligned and 4 bytes off: the word paths that
    # realign levels in registers, striding over many tiles
    for gmis in (False, True):
        print(f"[case] capped qsgd, levels at byte offsets, misaligned gradients={gmis}",
              flush=True)
        gb_dev = [gu.dev(g, gmis) for g in gs]
        bufs = [torch.full((n + 8,), 99, dtype=torch.int8, device=gu.DEV) for _ in range(W)]
        lvb = [bufs[w][1 + w % 3:1 + w % 3 + n] for w in range(W)]
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(gb_dev[w], norm, s, seed, w, lvb[w])
        sums_b = gu.empty(n, torch.int32, fill=-7)
        out_b = gu.empty(n, torch.float32, fill=float("nan"))
        gcq.qsgd_dequant_sum(lvb, norm, s, out_b, sums=sums_b)
        gu.sync()
        for w in range(W):
            check(np.array_equal(gu.host(lvb[w]), lv_or[w]), f"qsgd byte-offset levels worker {w}")
            hb = gu.host(bufs[w])
            check(np.all(hb[:1 + w % 3] == 99) and np.all(hb[1 + w % 3 + n:] == 99),
                  f"qsgd byte-offset levels: bytes outside the view, worker {w}")
        check(np.array_equal(gu.host(sums_b), s_or), "qsgd byte-offset level sums")
        check(np.array_equal(gu.host(out_b), d_or), "qsgd byte-offset dequantized")
    idx = oracle.randk_indices(n, 5000, 3)
    gk = gu.empty(5000, torch.float32)
    gcq.gather_f32(g_dev[0], gu.dev(idx), gk)
    dense = gu.empty(n, torch.float32, fill=float("nan"))
    gcq.qsgd_dequant_sum([gu.dev(q[:5000].copy()) for q in lv_or], norm, s, dense,
                         scatter_idx=gu.dev(idx), dense_n=n)
    gu.sync()
    check(np.array_equal(gu.host(gk), oracle.gather(gs[0], idx)), "gather")
    sk = oracle.level_sum([q[:5000].copy() for q in lv_or])
    check(np.array_equal(gu.host(dense),
                         oracle.scatter_dense(oracle.qsgd_dequantize(sk, norm_or, s), idx, n)),
          "scatter-dequantize")
    # the one-call GRandK step: one gather workgroup striding, a capped fill
    # (all of it beside the draw at n = 200,003; split between the first two
    # launches at n = 2,000,003)
    for n, K in ((200_003, 7_001), (2_000_003, 150)):
        capped_grandk_step(n, K)
    print("OK", flush=True)


def capped_grandk_step(n, K):
    print(f"[case] capped grandk_mn_step n={n} K={K}", flush=True)
    W, s, seed = 8, 7, 9
    gs = [si.normal_f32(500 + w, n, 0.01) for w in range(W)]
    g_dev = [gu.dev(g) for g in gs]
    idx = gu.empty(K, torch.int32)
    sums = gu.empty(K, torch.int32)
    dense = gu.empty(n, torch.float32, fill=float("nan"))
    ws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=gu.DEV)
    gcq.grandk_mn_step(g_dev, K, seed, s, idx, dense, ws, sums=sums)
    gu.sync()
    idx_or = oracle.randk_indices(n, K, seed)
    gk = [oracle.gather(g, idx_or) for g in gs]
    nrm = oracle.maxnorm(gk)
    S = oracle.level_sum([oracle.qsgd_quantize(g, nrm, s, seed, w) for w, g in enumerate(gk)])
    check(np.array_equal(gu.host(idx, np.uint32), idx_or), "grandk_mn_step indices")
    check(np.array_equal(gu.host(sums), S), "grandk_mn_step sums")
    check(np.array_equal(gu.host(dense), oracle.scatter_dense(oracle.qsgd_dequantize(S, nrm, s), idx_or, n)),
          f"grandk_mn_step dense n={n} K={K}")


if __name__ == "__main__":
    main()
