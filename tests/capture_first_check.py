"""A HIP graph captured in a fresh process before any eager call into the
library, so that the launch paths' one-time queries (each capped kernel's
own LDS, the device's LDS size) first run while the stream is capturing.
The capture must succeed, and every replay must match the oracle bit for
bit. Exits 0 and prints OK when it does; prints the failing case otherwise.
"""
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
    gcq.load()
    n, W, s, seed, thr = 100_003, 4, 127, 5, 0.05
    g_dev = [gu.empty(n, torch.float32) for _ in range(W)]
    r_dev = [torch.zeros(n, dtype=torch.float32, device=gu.DEV) for _ in range(W)]
    c2 = [gu.empty(gcq.gc_compressed_2bit_words(n), torch.int32) for _ in range(W)]
    c3 = [gu.empty(gcq.gc_compressed_ternary_words(n), torch.int32) for _ in range(W)]
    out2, out3 = gu.empty(n, torch.float32), gu.empty(n, torch.float32)
    norm = torch.empty(1, dtype=torch.float32, device=gu.DEV)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=gu.DEV)
    levels = [gu.empty(n, torch.int8) for _ in range(W)]
    sums, out = gu.empty(n, torch.int32), gu.empty(n, torch.float32)
    gu.sync()

    def step():
        for w in range(W):
            gcq.compress_2bit(g_dev[w], r_dev[w], -thr, thr, c2[w])
        gcq.decompress_2bit_sum(c2, n, out2)
        for w in range(W):
            gcq.compress_ternary(g_dev[w], r_dev[w], -thr, thr, c3[w])
        gcq.decompress_ternary_sum(c3, n, out3)
        gcq.qsgd_global_maxnorm(g_dev, norm, ws)
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(g_dev[w], norm, s, seed, w, levels[w])
        gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)

    print("[case] capture before any eager library call", flush=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step()
    gu.sync()
    r_or = [np.zeros(n, np.float32) for _ in range(W)]
    for t in range(3):
        print(f"[case] replay {t}", flush=True)
        grads = [si.normal_f32(si.grad_seed(w, 70 + t), n, 0.05) for w in range(W)]
        for d, a in zip(g_dev, grads):
            d.copy_(torch.from_numpy(a))
        for buf in (*c2, *c3, *levels, sums):
            buf.fill_(-1)
        for buf in (out2, out3, out, norm):
            buf.fill_(float("nan"))
        gu.sync()
        graph.replay()
        gu.sync()
        # the graph compresses twice per replay (2-bit, then ternary on the
        # residual the 2-bit pass left)
        q2 = [oracle.quantize_2bit(grads[w], r_or[w], -thr, thr) for w in range(W)]
        for w in range(W):
            check(np.array_equal(gu.host(c2[w], np.uint32), q2[w]), f"replay {t} 2-bit block {w}")
        check(np.array_equal(gu.host(out2).view(np.uint32),
                             oracle.dequantize_2bit_sum(q2, n).view(np.uint32)),
              f"replay {t} 2-bit sum")
        q3 = [oracle.quantize_ternary(grads[w], r_or[w], -thr, thr) for w in range(W)]
        for w in range(W):
            check(np.array_equal(gu.host(c3[w], np.uint32), q3[w]), f"replay {t} ternary block {w}")
            check(np.array_equal(gu.host(r_dev[w]).view(np.uint32), r_or[w].view(np.uint32)),
                  f"replay {t} residual {w}")
        check(np.array_equal(gu.host(out3).view(np.uint32),
                             oracle.dequantize_ternary_sum(q3, n).view(np.uint32)),
              f"replay {t} ternary sum")
        nrm = oracle.maxnorm(grads)
        check(gu.host(norm)[0] == nrm, f"replay {t} norm")
        lv = [oracle.qsgd_quantize(g, nrm, s, seed, w) for w, g in enumerate(grads)]
        for w in range(W):
            check(np.array_equal(gu.host(levels[w]), lv[w]), f"replay {t} levels {w}")
        S = oracle.level_sum(lv)
        check(np.array_equal(gu.host(sums), S), f"replay {t} sums")
        check(np.array_equal(gu.host(out).view(np.uint32),
                             oracle.qsgd_dequantize(S, nrm, s).view(np.uint32)),
              f"replay {t} dequantized")
    print("OK", flush=True)


if __name__ == "__main__":
    main()
