#!/usr/bin/env python3
"""Benchmark of the gradient-quantization hot path on one MI355X.

Step (the workload of the headline metric): one data-parallel step of 2-bit
error-feedback compression on a ResNet-50-sized flat fp32 gradient,
25,557,032 values per worker, W = 8 simulated workers, thresholds +-0.01:
compress_2bit for each worker (residual carried across steps), then
decompress_2bit_sum of the 8 blocks into one fp32 array in worker order.
`value` is the step's algorithmic bytes over its wall time on the device.

The metric's second half, QSGD-MN elements/s, is measured in the same run on
its own workload (VGG16-sized heavy-tailed gradient, 138,357,544 values x 8
workers, s = 127): global max-norm, 8 quantizes, level sum + dequantize.

Inputs are synthetic (seeded N(0, sigma^2) fp32, see synthetic_inputs.py) and
resident in HBM before timing starts. Per-kernel durations come from HIP
events recorded on the stream the kernels are launched on.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import platform
import re
import statistics
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
N_C2 = 25_557_032              # ResNet-50 parameter count
W_C2 = 8
THR_C2 = 0.01
SIGMA_C2 = 0.01
N_C3 = 138_357_544             # VGG16 parameter count
W_C3 = 8
S_C3 = 127
SIGMA_C3 = 0.02

PROFILE_TRAFFIC = ROOT / "profiles" / "hbm_traffic_resnet50_vgg16.md"
PROFILE_STATS = ROOT / "profiles" / "kernel_stats_resnet50_vgg16.md"
PROFILE_STATS_EXTRA = ROOT / "profiles" / "kernel_stats_bert_multitensor_grandk_ternary.md"
PROFILE_VALU = ROOT / "profiles" / "valu_busy_all_workloads.md"
KERNEL_SOURCES = [ROOT / "gradient_compression_quantize_amd" / "csrc" / f
                  for f in ("gcq_internal.h", "occupancy.h", "threshold_codes.h", "twobit.hip",
                            "ternary.hip", "qsgd.hip")]

# The rocprofv3 runs the committed summaries come from (run from the repo
# root; prof_out/ is scratch output, not kept in the repository).
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -T -d prof_out/prof_bench -o bench "
             "--output-format csv -- python3 -u bench.py --steps 20 --warmup 5 --qsgd-steps 5 "
             "--skip-cpu-baseline --skip-extra",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -T -d prof_out/pmc_fetch -o fetch --output-format csv "
             "-- python3 -u bench.py --steps 3 --warmup 1 --qsgd-steps 1 --skip-cpu-baseline "
             "--skip-extra",
    "write": "rocprofv3 --pmc WRITE_SIZE -T -d prof_out/pmc_write -o write --output-format csv "
             "-- python3 -u bench.py --steps 3 --warmup 1 --qsgd-steps 1 --skip-cpu-baseline "
             "--skip-extra",
    "trace_extra": "rocprofv3 --kernel-trace --stats -T -d prof_out/prof_extra -o extra "
                   "--output-format csv -- python3 -u bench.py --extras-only",
    "fetch_extra": "rocprofv3 --pmc FETCH_SIZE -T -d prof_out/pmc_fetch_extra -o fetch "
                   "--output-format csv -- python3 -u bench.py --extras-only --extra-steps 3",
    "write_extra": "rocprofv3 --pmc WRITE_SIZE -T -d prof_out/pmc_write_extra -o write "
                   "--output-format csv -- python3 -u bench.py --extras-only --extra-steps 3",
    "valu": "rocprofv3 --pmc VALUBusy SQ_INSTS_VALU SQ_INSTS_LDS -T -d prof_out/pmc_valu -o valu "
            "--output-format csv -- python3 -u bench.py --steps 3 --warmup 1 --qsgd-steps 1 "
            "--skip-cpu-baseline --skip-extra",
    "valu_extra": "rocprofv3 --pmc VALUBusy SQ_INSTS_VALU SQ_INSTS_LDS -T -d prof_out/pmc_valu_extra "
                  "-o valu --output-format csv -- python3 -u bench.py --extras-only --extra-steps 3",
    "cal_fetch": "rocprofv3 --pmc FETCH_SIZE -T -d prof_out/pmc_cal_fetch -o cal "
                 "--output-format csv -- python3 -u bench.py --calibrate-copy",
    "cal_write": "rocprofv3 --pmc WRITE_SIZE -T -d prof_out/pmc_cal_write -o cal "
                 "--output-format csv -- python3 -u bench.py --calibrate-copy",
    "ceilings": "rocprofv3 --kernel-trace --stats -T -d prof_out/prof_ceilings -o ceil "
                "--output-format csv -- python3 -u bench.py --calibrate-ceilings",
    "summary": "python3 bench.py --summarize-profiles prof_out",
}
PROFILE_CEILINGS = ROOT / "profiles" / "hbm_ceilings.md"
CEILING_SOURCES = [ROOT / "gradient_compression_quantize_amd" / "csrc" / f
                   for f in ("hbm_ceilings.hip", "occupancy.h")]
# Resident workgroups per CU each ceiling pattern is also timed at (0: what
# the kernel's registers allow); a mix's ceiling is its best pattern and cap.
CEILING_WG_PER_CU = (0, 3, 4, 5)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def compress_bytes(n: int) -> int:
    """Algorithmic HBM bytes of one compress_2bit call: read grad and residual,
    write residual (12 B per value) and the block of 3 + ceil(n/16) words."""
    return 12 * n + 4 * (3 + (n + 15) // 16)


def dequant_sum_bytes(n: int, W: int) -> int:
    """Read W packed blocks, write n fp32 values."""
    return 4 * W * (3 + (n + 15) // 16) + 4 * n


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--qsgd-steps", type=int, default=10)
    ap.add_argument("--skip-qsgd", action="store_true", help="time only the 2-bit step")
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--skip-extra", action="store_true",
                    help="skip the many-tensor, GlobalRandK, ternary and misaligned-buffer measurements")
    ap.add_argument("--extras-only", action="store_true",
                    help="only the many-tensor, GlobalRandK, ternary and misaligned-buffer measurements (profiling)")
    ap.add_argument("--extra-steps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU time budget of the oracle baseline sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device copy of 1 GiB (counter calibration)")
    ap.add_argument("--calibrate-ceilings", action="store_true",
                    help="only time the HBM ceiling kernels (plain streams with each hot-path "
                         "kernel's access mix) and print their rates")
    ap.add_argument("--skip-ceilings", action="store_true",
                    help="do not time the HBM ceiling kernels (no frac_of_ceiling fields)")
    ap.add_argument("--ceiling-steps", type=int, default=20)
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from rocprofv3 output under DIR")
    return ap.parse_args()


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES if sources is None else sources):
        h.update(f.read_bytes())
    return h.hexdigest()


def traffic_from_profile(kernel: str, profile: pathlib.Path | None = None,
                         key: str = "traffic_bytes_per_launch") -> int | None:
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters, if
    the committed measurement was taken on the current kernel sources."""
    profile = profile or PROFILE_TRAFFIC
    if not profile.exists():
        return None
    text = profile.read_text()
    m_h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]+)", text, re.M)
    m_b = re.search(rf"^{key}\[{kernel}\]:\s*([0-9]+)", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != kernel_source_hash():
        return None
    return int(m_b.group(1))


# VALU peak: 256 CUs x 64 lanes (four 16-lane SIMDs) x 2.4 GHz, one
# non-packed VALU instruction per lane per cycle.
VALU_PEAK_T_LANE_INSTS = 256 * 64 * 2.4e9 / 1e12


def valu_insts_from_profile(kernel: str) -> int | None:
    """SQ_INSTS_VALU (wave-level VALU instructions) per launch of `kernel`
    from the committed rocprofv3 summary, if taken on the current sources."""
    if not PROFILE_VALU.exists():
        return None
    text = PROFILE_VALU.read_text()
    m_h = re.search(r"^kernel_source_sha256:\s*([0-9a-f]+)", text, re.M)
    m_v = re.search(rf"^valu_insts_per_launch\[{kernel}\]:\s*([0-9]+)", text, re.M)
    if not (m_v and m_h) or m_h.group(1) != kernel_source_hash():
        return None
    return int(m_v.group(1))


def _read_counters(path: pathlib.Path):
    import csv
    import collections
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return per


def _read_counters_fewest_lds(path: pathlib.Path):
    """{kernel: [value per dispatch]} keeping, for each kernel, only the
    dispatches of the instantiation that declares the least LDS of its own
    (the counter CSV's LDS_Block_Size). The dequantize-sums declare more for
    run-time W than for compile-time W <= 8, so this keeps the W = 8
    launches of the workloads' steps and drops the many-worker runs'."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]][int(r.get("LDS_Block_Size") or 0)].append(float(r["Counter_Value"]))
    return {k: v[min(v)] for k, v in per.items()}


def copy_calibration(d: pathlib.Path):
    """(FETCH scale, WRITE scale, copy kernel, FETCH KiB, WRITE KiB) from the
    1 GiB device copy of --calibrate-copy: bytes = counter KiB x 1024 x
    scale. None without the two calibration passes."""
    if not (d / "pmc_cal_fetch").exists() or not (d / "pmc_cal_write").exists():
        return None
    cal_f = _read_counters(next((d / "pmc_cal_fetch").glob("*counter_collection.csv")))
    cal_w = _read_counters(next((d / "pmc_cal_write").glob("*counter_collection.csv")))
    copy_name = max(cal_w, key=lambda k: sum(cal_w[k]))
    copy_bytes = 4 << 28
    f_kib = sum(cal_f[copy_name]) / len(cal_f[copy_name])
    w_kib = sum(cal_w[copy_name]) / len(cal_w[copy_name])
    return copy_bytes / (f_kib * 1024), copy_bytes / (w_kib * 1024), copy_name, f_kib, w_kib


def _read_counters_by_name(path: pathlib.Path):
    """{kernel: {counter: [value per dispatch]}} from a rocprofv3 counter CSV,
    for each kernel only the dispatches of the instantiation that declares
    the least LDS of its own (as _read_counters_fewest_lds)."""
    import csv
    import collections
    per = collections.defaultdict(
        lambda: collections.defaultdict(lambda: collections.defaultdict(list)))
    for r in csv.DictReader(open(path)):
        per[r["Kernel_Name"]][int(r.get("LDS_Block_Size") or 0)][r["Counter_Name"]].append(
            float(r["Counter_Value"]))
    return {k: v[min(v)] for k, v in per.items()}


def summarize_valu(d: pathlib.Path) -> pathlib.Path | None:
    """profiles/ summary of VALUBusy / SQ_INSTS_VALU / SQ_INSTS_LDS per kernel."""
    files = [f for sub in ("pmc_valu", "pmc_valu_extra") if (d / sub).exists()
             for f in (d / sub).glob("*counter_collection.csv")]
    if not files:
        return None
    rows = {}
    for f in files:
        for k, cs in _read_counters_by_name(f).items():
            rows.setdefault(k, cs)
    lines = [
        "# VALU activity per kernel from rocprofv3 counters",
        "",
        "Commands (repo root):",
        "",
        f"    {PROFILE_COMMANDS['valu']}",
        f"    {PROFILE_COMMANDS['valu_extra']}",
        f"    {PROFILE_COMMANDS['summary']}",
        "",
        "VALUBusy is rocprofv3's derived metric 100 * sum(SQ_ACTIVE_INST_VALU) / CU_NUM / "
        "max(GRBM_GUI_ACTIVE): the share of the kernel's GPU time in which the CUs issue vector "
        "ALU work. SQ_INSTS_VALU and SQ_INSTS_LDS count wave-level instructions per dispatch. "
        "A kernel near its HBM roofline shows a low VALUBusy; one bound by its arithmetic "
        "shows a high one. Each row counts one instantiation of its kernel, the one that "
        "declares the least LDS of its own: for the dequantize-sums the W = 8 launches, not "
        "the many-worker runs' run-time-W ones.",
        "",
        "| kernel | dispatches | VALUBusy % | SQ_INSTS_VALU per dispatch | SQ_INSTS_LDS per dispatch |",
        "|---|---|---|---|---|",
    ]
    mean = lambda v: sum(v) / len(v) if v else float("nan")  # noqa: E731
    for k in sorted(rows, key=lambda k: -mean(rows[k].get("VALUBusy", [0]))):
        cs = rows[k]
        lines.append(f"| {k} | {len(cs.get('SQ_INSTS_VALU', []))} | {mean(cs.get('VALUBusy', [])):.1f} | "
                     f"{mean(cs.get('SQ_INSTS_VALU', [])):,.0f} | {mean(cs.get('SQ_INSTS_LDS', [])):,.0f} |")
    lines += ["", "Machine-readable (bench.py reads these while the kernel sources are unchanged):",
              "", f"kernel_source_sha256: {kernel_source_hash()}"]
    lines += [f"valu_insts_per_launch[{k}]: {int(round(mean(rows[k]['SQ_INSTS_VALU'])))}"
              for k in sorted(rows) if rows[k].get("SQ_INSTS_VALU")]
    lines.append("")
    PROFILE_VALU.write_text("\n".join(lines))
    return PROFILE_VALU


def ceiling_kernel_bytes() -> dict:
    """Bytes per launch of each ceiling kernel at the sizes measure_ceilings
    uses (the workloads rounded down to whole 16384-value quanta)."""
    Q = 16384
    n2, n3 = N_C2 // Q * Q, N_C3 // Q * Q
    nt = N_C2 // 81920 * 81920
    return {
        "ceil_read_chunked_kernel": (4 * W_C3 * n3, "read, chunked (8 buffers per launch)"),
        "ceil_read_tile_kernel": (4 * n3, "read, one tile per wave (1 buffer per launch)"),
        "ceil_levelsum_mix_kernel": ((W_C3 + 8) * n3, "level-sum mix (W = 8)"),
        "ceil_quantize_sum_mix_kernel": ((4 * W_C3 + 8) * n3, "fused quantize-sum mix (W = 8)"),
        "ceil_quantize_mix_kernel": (5 * n3, "quantize mix"),
        "ceil_write_tile_kernel": (4 * n2, "write, one tile per wave"),
        "ceil_write_stride_kernel": (4 * n2, "write, grid-stride"),
        "ceil_compress_mix_kernel": (compress_bytes(n2), "compress mix"),
        "ceil_dequant_tile_kernel": (dequant_sum_bytes(n2, W_C2), "dequantize-sum mix, the kernel's pattern"),
        "ceil_dequant_wide_kernel": (dequant_sum_bytes(n2, W_C2), "dequantize-sum mix, wide reads"),
        "ceil_dequant_burst_kernel": (dequant_sum_bytes(n2, W_C2), "dequantize-sum mix, workgroup bursts"),
        "ceil_dequant_ternary_kernel": (4 * W_C2 * (3 + nt // 20) + 4 * nt,
                                        "ternary dequantize-sum mix (at n = %d)" % nt),
    }


def summarize_ceilings(d: pathlib.Path) -> pathlib.Path | None:
    """profiles/hbm_ceilings.md from the kernel trace of --calibrate-ceilings:
    the average duration of each ceiling kernel at each occupancy cap.
    measure_ceilings times every pattern once per cap of CEILING_WG_PER_CU,
    in that order, with the same number of launches each time, so a
    kernel's launches in time order fall into that many equal runs, one per
    cap (the trace's LDS_Block_Size shows the kernel's own LDS only). A
    kernel timed uncapped only (the burst pattern) has one run."""
    import csv
    root = d / "prof_ceilings"
    files = list(root.glob("*kernel_trace.csv")) if root.exists() else []
    if not files:
        return None
    launches: dict = {}
    for r in csv.DictReader(open(files[0])):
        name = r["Kernel_Name"].split("(")[0].split("::")[-1].strip()
        if name.startswith("ceil_"):
            launches.setdefault(name, []).append(
                (int(r["Start_Timestamp"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
    durs: dict = {}
    for name, v in launches.items():
        v.sort()
        caps = CEILING_WG_PER_CU if name != "ceil_dequant_burst_kernel" else (0,)
        if len(v) % len(caps):
            raise ValueError(f"{name}: {len(v)} launches do not split into {len(caps)} caps")
        m = len(v) // len(caps)
        for i, cap in enumerate(caps):
            durs[(name, cap)] = [us for _, us in v[i * m:(i + 1) * m]]
    Q = 16384
    lines = [
        "# HBM ceilings of the hot path's access mixes (rocprofv3 kernel trace)",
        "",
        "Commands (repo root):",
        "",
        f"    {PROFILE_COMMANDS['ceilings']}",
        f"    {PROFILE_COMMANDS['summary']}",
        "",
        "Plain streaming kernels (`gradient_compression_quantize_amd/csrc/hbm_ceilings.hip`, "
        "built into `libgcq_ceilings.so`) that move exactly the bytes of one hot-path kernel in "
        "its tile shapes, with trivial arithmetic in place of the quantization. Sizes: "
        f"{N_C3 // Q * Q:,} values (VGG16, rounded down to a multiple of {Q}) for read, level sum "
        f"and quantize; {N_C2 // Q * Q:,} (ResNet-50, rounded) for write, compress and the "
        "dequantize-sum. Each launch rotates over buffer sets larger than the Infinity Cache. "
        "Every pattern runs with what its registers allow per CU (\"-\") and held by an LDS "
        f"reservation to {', '.join(str(c) for c in CEILING_WG_PER_CU if c)} resident "
        "workgroups per CU. `bench.py` times the same kernels live with events in every default "
        "run and reports each hot-path kernel's rate over its mix's best rate as "
        "`frac_of_ceiling`.",
        "",
        "| kernel | mix | workgroups per CU | calls | average us | bytes per launch | GB/s | "
        "% of 8 TB/s |",
        "|---|---|---|---|---|---|---|---|",
    ]
    for k, (nb, what) in ceiling_kernel_bytes().items():
        for cap in sorted(c for (name, c) in durs if name == k):
            v = durs[(k, cap)]
            us = statistics.mean(v)
            gbs = nb / (us * 1e-6) / 1e9
            lines.append(f"| {k} | {what} | {cap or '-'} | {len(v)} | {us:.2f} | {nb:,} | "
                         f"{gbs:,.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} |")
    lines += ["", f"ceiling_source_sha256: {kernel_source_hash(CEILING_SOURCES)}", ""]
    PROFILE_CEILINGS.write_text("\n".join(lines))
    return PROFILE_CEILINGS


PROFILE_GRANDK = ROOT / "profiles" / "grandk_step_critical_path.md"


def summarize_grandk_path(d: pathlib.Path) -> pathlib.Path | None:
    """profiles/grandk_step_critical_path.md: the launches of the one-call
    GlobalRandK-MN step at the ResNet-50 size and at n = 2^20 (the chain with
    almost no fill), and each stage run alone, from the kernel trace of the
    extras run."""
    import csv
    files = list((d / "prof_extra").glob("*kernel_trace.csv")) if (d / "prof_extra").exists() else []
    if not files:
        return None
    rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Start_Timestamp"]))
    ts = lambda r, k: int(r[k + "_Timestamp"])  # noqa: E731
    dur = lambda r: (ts(r, "End") - ts(r, "Start")) / 1e3  # noqa: E731
    med = lambda v: statistics.median(v) if v else float("nan")  # noqa: E731
    names = ("grandk_draw_fill_kernel", "grandk_gather_fill_kernel",
             "grandk_quantize_scatter_kernel")
    steps = [rows[i:i + 3] for i in range(len(rows) - 2)
             if all(rows[i + j]["Kernel_Name"].startswith(names[j]) for j in range(3))]
    if not steps:
        return None
    # the full-size steps have the larger launch-1 grid (more fill workgroups)
    grids = sorted({int(t[0]["Grid_Size_X"]) for t in steps})
    big = [t for t in steps if int(t[0]["Grid_Size_X"]) == grids[-1]]
    small = [t for t in steps if int(t[0]["Grid_Size_X"]) == grids[0]] if len(grids) > 1 else []

    def launch_rows(group):
        l1, l2, l3 = ([dur(t[j]) for t in group] for j in range(3))
        g12 = [(ts(t[1], "Start") - ts(t[0], "End")) / 1e3 for t in group]
        g23 = [(ts(t[2], "Start") - ts(t[1], "End")) / 1e3 for t in group]
        whole = [(ts(t[2], "End") - ts(t[0], "Start")) / 1e3 for t in group]
        nxt = [(ts(group[i + 1][0], "Start") - ts(group[i][0], "Start")) / 1e3
               for i in range(len(group) - 1)]
        return [med(l1), med(g12), med(l2), med(g23), med(l3), med(whole), med(nxt), len(group)]

    by = lambda name: [dur(r) for r in rows if r["Kernel_Name"].startswith(name)]  # noqa: E731
    n, K, W = N_C2, 10_000, W_C2
    draw = by("grandk_indices_lds_kernel")
    fill = by("fill_zero_kernel")
    gather = by("gather_kernel")
    # the separate-call step's quantizes are the smallest qsgd_quantize launches
    qrows = [r for r in rows if r["Kernel_Name"].startswith("qsgd_quantize")
             and "sum" not in r["Kernel_Name"]]
    gmin = min((int(r["Grid_Size_X"]) for r in qrows), default=0)
    quant = [dur(r) for r in qrows if int(r["Grid_Size_X"]) == gmin]
    scatter = by("qsgd_dequant_scatter_kernel")
    ceil_gbs = None
    if PROFILE_CEILINGS.exists():
        # the best write-tile row over the occupancy caps
        rates = [float(m.group(3).replace(",", "")) for m in re.finditer(
            r"^\| ceil_write_tile_kernel \|.*?\| ([0-9.]+) \| ([0-9,]+) \| ([0-9,]+) \|",
            PROFILE_CEILINGS.read_text(), re.M)]
        if rates:
            ceil_gbs = max(rates)
    fill_floor = 4 * n / (ceil_gbs * 1e3) if ceil_gbs else None  # us
    B = launch_rows(big)
    S = launch_rows(small) if small else [float("nan")] * 8
    what = ["1 `grandk_draw_fill_kernel`: the K-index draw in one workgroup (Philox targets, "
            "LDS chains), beside the first share of the dense zero fill",
            "gap", "2 `grandk_gather_fill_kernel`: W x K gathers and partial maxima, beside the "
            "rest of the fill", "gap",
            "3 `grandk_quantize_scatter_kernel`: norm, levels, sums, dequantize, scatter",
            "first launch's start to last launch's end",
            "one step's start to the next step's start", "steps traced"]
    lines = [
        "# GlobalRandK-MN step: per-launch critical path (rocprofv3 kernel trace)",
        "",
        "Commands (repo root):",
        "",
        f"    {PROFILE_COMMANDS['trace_extra']}",
        f"    {PROFILE_COMMANDS['summary']}",
        "",
        f"Workload: K = {K}, W = {W}, s = 7, at n = {n:,} (ResNet-50) and at n = 1,048,576 "
        "(the same chain of draw, gathers, norm, quantize and scatter with a 4 MB fill instead "
        "of a 102 MB one). `grandk_mn_step` is three launches on one stream. Durations are "
        "medians over the trace's launches (eager calls and graph replays together); the "
        "profiler adds latency of its own between launches, so the spans are longer than the "
        "graph-timed `grandk_mn.ms_per_step` and `chain_ms_per_step` of the bench line.",
        "",
        f"| grandk_mn_step | n = {n:,}, us | n = 1,048,576, us |",
        "|---|---|---|",
    ]
    for k in range(7):
        lines.append(f"| {what[k]} | {B[k]:.2f} | {S[k]:.2f} |")
    lines.append(f"| {what[7]} | {B[7]} | {S[7]} |")
    lines += [
        "",
        "| stage alone (the separate-call step at the full size) | kernel | median us |",
        "|---|---|---|",
        f"| the draw | `grandk_indices_lds_kernel` | {med(draw):.2f} |",
        f"| the dense zero fill, {4 * n:,} B | `fill_zero_kernel` | {med(fill):.2f} |",
        f"| one worker's gather of K values | `gather_kernel` | {med(gather):.2f} |",
        f"| one worker's quantize of K values | `qsgd_quantize*` (K-sized launches) | "
        f"{med(quant):.2f} |",
        f"| level sum, dequantize, scatter | `qsgd_dequant_scatter_kernel` | {med(scatter):.2f} |",
        "",
    ]
    if fill_floor:
        lines += [f"Fill floor: {4 * n:,} B at the measured write ceiling "
                  f"({ceil_gbs:,.0f} GB/s, `profiles/hbm_ceilings.md`) = {fill_floor:.1f} us.", ""]
    lines += grandk_traffic_lines(d, names, n)
    lines += [
        "Reading:",
        "",
        "- At n = 1,048,576 the fill is negligible, so that column is the chain itself: the "
        "draw in launch 1, then the gathers, then norm -> quantize -> scatter, with two launch "
        "gaps between them. The full-size step costs that chain plus the part of the fill that "
        "does not hide beside it.",
        "- Launch 1 lasts about as long as the draw run alone: the draw only touches LDS, so "
        "the fill beside it runs at full speed and costs the step nothing extra.",
        "- Launch 2 is where the fill and the gathers meet: the gathers' scattered reads slow "
        "while the fill's writes drain, and the fill slows beside them.",
        "- Launch 3 must follow the whole fill (its scatter lands anywhere in dense).",
        "",
    ]
    PROFILE_GRANDK.write_text("\n".join(lines))
    return PROFILE_GRANDK


def grandk_traffic_lines(d: pathlib.Path, names, n: int) -> list:
    """HBM bytes of each launch of the full-size GlobalRandK step from the
    FETCH_SIZE and WRITE_SIZE passes over the extras run, calibrated on the
    device copy; [] without those passes."""
    import csv
    cal = copy_calibration(d)
    if cal is None or not (d / "pmc_fetch_extra").exists() or not (d / "pmc_write_extra").exists():
        return []
    f_scale, w_scale = cal[0], cal[1]

    def per_launch(sub, scale):
        rows = sorted(csv.DictReader(open(next((d / sub).glob("*counter_collection.csv")))),
                      key=lambda r: int(r["Dispatch_Id"]))
        rows = [r for r in rows if r["Kernel_Name"].startswith(names)]
        steps = [rows[i:i + 3] for i in range(len(rows) - 2)
                 if all(rows[i + j]["Kernel_Name"].startswith(names[j]) for j in range(3))]
        if not steps:
            return None
        big = max(int(t[0]["Grid_Size"]) for t in steps)
        steps = [t for t in steps if int(t[0]["Grid_Size"]) == big]
        return [statistics.median(float(t[j]["Counter_Value"]) for t in steps) * 1024 * scale
                for j in range(3)], len(steps)

    f, w = per_launch("pmc_fetch_extra", f_scale), per_launch("pmc_write_extra", w_scale)
    if not f or not w:
        return []
    (fb, nf), (wb, nw) = f, w
    tot = sum(fb) + sum(wb)
    out = [
        f"HBM bytes of the full-size step (medians over {min(nf, nw)} steps; one counter per "
        "run, calibrated on a 1 GiB device copy):",
        "",
        f"    {PROFILE_COMMANDS['fetch_extra']}",
        f"    {PROFILE_COMMANDS['write_extra']}",
        "",
        "| launch | read (FETCH_SIZE) | written (WRITE_SIZE) |",
        "|---|---|---|",
    ]
    for j in range(3):
        out.append(f"| {j + 1} `{names[j]}` | {fb[j]:,.0f} B | {wb[j]:,.0f} B |")
    K, W = 10_000, W_C2
    out += [f"| step | {sum(fb):,.0f} B | {sum(wb):,.0f} B |", "",
            f"The step moves {tot:,.0f} B, {tot / (4 * n):.3f}x its {4 * n:,} B of dense "
            f"output. Nearly all the reads are launch 2's gathers: W x K = {W * K:,} random "
            f"4-byte values, each costing a 128-byte line ({W * K * 128:,} B). The writes "
            "are the dense output, the gathered values and the scattered lines.", "",
            "Machine-readable (bench.py reads this while the kernel sources are unchanged):", "",
            f"kernel_source_sha256: {kernel_source_hash()}",
            f"traffic_bytes_per_step[grandk_mn_step]: {int(round(tot))}", ""]
    return out


def summarize_profiles(out_dir: str) -> None:
    """Write the profiles/ summaries whose rocprofv3 CSV output is under
    out_dir (each summary needs only its own runs)."""
    import csv
    d = pathlib.Path(out_dir)
    wrote = []
    c = summarize_ceilings(d)
    if c:
        wrote.append(c)
    gk = summarize_grandk_path(d)
    if gk:
        wrote.append(gk)
    if not (d / "pmc_cal_fetch").exists():
        print("wrote " + ", ".join(str(w) for w in wrote))
        return
    n2, W2, n3, W3 = N_C2, W_C2, N_C3, W_C3
    algo = {
        "compress_2bit_vec_kernel": (8 * n2, 4 * n2 + 4 * (3 + (n2 + 15) // 16)),
        "decompress_2bit_vec_kernel": (4 * W2 * (3 + (n2 + 15) // 16), 4 * n2),
        "maxabs_partial_kernel": (4 * W3 * n3, 0),
        "qsgd_quantize_kernel": (4 * n3, n3),
        "qsgd_dequant_sum_kernel": (W3 * n3, 8 * n3),
        "qsgd_quantize_sum_kernel": (4 * W3 * n3, 8 * n3),
    }
    f_scale, w_scale, copy_name, f_kib, w_kib = copy_calibration(d)
    copy_bytes = 4 << 28
    fetch = _read_counters_fewest_lds(next((d / "pmc_fetch").glob("*counter_collection.csv")))
    write = _read_counters_fewest_lds(next((d / "pmc_write").glob("*counter_collection.csv")))
    sizes = [int(v) for v in __import__("synthetic_inputs").bert_base_sizes()]
    if (d / "pmc_fetch_extra").exists() and (d / "pmc_write_extra").exists():
        fx = _read_counters_fewest_lds(
            next((d / "pmc_fetch_extra").glob("*counter_collection.csv")))
        wx = _read_counters_fewest_lds(
            next((d / "pmc_write_extra").glob("*counter_collection.csv")))
        tw = ternary_words(n2)
        extra_algo = {
            "compress_2bit_multi_kernel": (8 * sum(sizes), multi_bytes(sizes) - 8 * sum(sizes)),
            "compress_ternary_vec_kernel": (8 * n2, 4 * n2 + 4 * tw),
            "decompress_ternary_vec_kernel": (4 * W2 * tw, 4 * n2),
        }
        for k, ab in extra_algo.items():
            if k in fx and k in wx:
                fetch[k], write[k] = fx[k], wx[k]
                algo[k] = ab
    lines = [
        "# HBM traffic per launch from rocprofv3 counters",
        "",
        "Workloads: the 2-bit step on the ResNet-50-sized flat gradient "
        f"({n2:,} fp32 values, {W2} workers, thresholds +-0.01), the QSGD-MN step on the "
        f"VGG16-sized gradient ({n3:,} fp32 values, {W3} workers, s = 127), the "
        f"many-tensor compress over the BERT-Base list (198 tensors, {sum(sizes):,} values), "
        "and the 2-bit step's workload with the codes packed five per byte (ternary).",
        "",
        "Commands (repo root, one counter per run):",
        "",
        *[f"    {PROFILE_COMMANDS[k]}" for k in ("fetch", "write", "fetch_extra", "write_extra",
                                                 "cal_fetch", "cal_write", "summary")],
        "",
        "Calibration: a plain device copy of 1 GiB (`bench.py --calibrate-copy`, "
        f"kernel `{copy_name}`) reads and writes {copy_bytes:,} bytes. Its counters read "
        f"FETCH_SIZE = {f_kib:,.1f} KiB and WRITE_SIZE = {w_kib:,.1f} KiB per dispatch, so "
        f"bytes = FETCH_SIZE x 1024 x {f_scale:.4f} and WRITE_SIZE x 1024 x {w_scale:.4f}.",
        "",
        "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | "
        "algorithmic bytes | ratio |",
        "|---|---|---|---|---|---|---|",
    ]
    machine = []
    for k, (ar, aw) in algo.items():
        if k not in fetch or k not in write:
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write[k]) / len(write[k])
        hb = fk * 1024 * f_scale + wk * 1024 * w_scale
        lines.append(f"| {k} | {len(fetch[k])} | {fk:,.1f} | {wk:,.1f} | {hb:,.0f} | "
                     f"{ar + aw:,} | {hb / (ar + aw):.4f} |")
        machine.append(f"traffic_bytes_per_launch[{k}]: {int(round(hb))}")
    lines += ["", "Algorithmic bytes: compress reads grad and residual and writes residual and "
              "the block (12 n + 4 (3 + ceil(n/16)), or 4 (3 + ceil(n/20)) for the ternary "
              "block); dequantize-sum reads W blocks and writes "
              "n fp32; max-norm reads W n fp32; quantize reads n fp32 and writes n int8; the "
              "level sum reads W n int8 and writes n int32 + n fp32; the fused quantize-sum "
              "reads W n fp32 and writes n int32 + n fp32. The dequantize-sum rows count the "
              "W = 8 launches only (told apart from the many-worker runs' run-time-W "
              "instantiation by the LDS the kernel declares).", "",
              "Machine-readable (bench.py reads these while the kernel sources are unchanged):",
              "", f"kernel_source_sha256: {kernel_source_hash()}", *machine, ""]
    PROFILE_TRAFFIC.write_text("\n".join(lines))

    stats = list(csv.DictReader(open(next((d / "prof_bench").glob("*kernel_stats.csv")))))
    lines = [
        "# Kernel durations from rocprofv3 (kernel trace)",
        "",
        "Command (repo root):",
        "",
        f"    {PROFILE_COMMANDS['trace']}",
        f"    {PROFILE_COMMANDS['summary']}",
        "",
        "The 2-bit step (8 x compress_2bit + decompress_2bit_sum W=8) runs 5 warm-up, 20 timed, "
        "20 kernel-timing and 20 graph-replayed steps; the QSGD-MN step runs 2 warm-up and 5 "
        "timed steps, then 1 + 5 steps of its fused form (max-norm + qsgd_quantize_sum).",
        "",
        "| kernel | calls | average us | min us | max us | share of GPU time |",
        "|---|---|---|---|---|---|",
    ]
    for r in stats:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f}% |")
    comp = next((r for r in stats if r["Name"] == "compress_2bit_vec_kernel"), None)
    if comp:
        us = float(comp["AverageNs"]) / 1e3
        gbs = compress_bytes(n2) / (us * 1e-6) / 1e9
        lines += ["", f"compress_2bit at {n2:,} values: {compress_bytes(n2):,} algorithmic bytes "
                  f"in {us:.2f} us = {gbs:,.0f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of "
                  f"{HBM_PEAK_GBS:,.0f} GB/s."]
    lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
    PROFILE_STATS.write_text("\n".join(lines))
    wrote += [PROFILE_TRAFFIC, PROFILE_STATS]
    extra = list((d / "prof_extra").glob("*kernel_stats.csv")) if (d / "prof_extra").exists() else []
    if extra:
        stats = list(csv.DictReader(open(extra[0])))
        lines = [
            "# Kernel durations from rocprofv3: many-tensor compress, GlobalRandK, ternary, "
            "misaligned buffers, many workers",
            "",
            "Command (repo root):",
            "",
            f"    {PROFILE_COMMANDS['trace_extra']}",
            f"    {PROFILE_COMMANDS['summary']}",
            "",
            f"Many-tensor: compress_2bit_multi over the BERT-Base list (198 tensors, "
            f"{sum(sizes):,} values, {multi_bytes(sizes):,} algorithmic bytes per call). "
            "GlobalRandK-MN: n = 25,557,032, K = 10000, W = 8, s = 7; eager steps, then graph "
            "replays of the whole step. Ternary: the 2-bit step's workload (n = 25,557,032, "
            "W = 8, thresholds +-0.01) with compress_ternary + decompress_ternary_sum; 3 "
            "warm-up, then timed, kernel-timing and graph-replayed steps. Misaligned "
            "buffers: the 2-bit and ternary compress and W = 8 dequantize-sum at the "
            "ResNet-50 size, and the QSGD-MN max-norm, quantize, level sum and fused "
            "quantize-sum at the VGG16 size, each on buffers 4 bytes off 16-byte alignment "
            "(the *_dword_kernel rows) and on aligned buffers. Many workers: the 2-bit and "
            "ternary dequantize-sums at W = 16 and 64 (the run-time-W kernels) at the "
            "ResNet-50 size. GlobalRandK also runs at n = 1,048,576 (the chain alone), and "
            "the W = 8 dequantize-sum rows mix the workloads above, so their averages are "
            "not one workload's.",
            "",
            "| kernel | calls | average us | min us | max us | share of GPU time |",
            "|---|---|---|---|---|---|",
        ]
        for r in stats:
            lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.2f}% |")
        m = next((r for r in stats if r["Name"] == "compress_2bit_multi_kernel"), None)
        if m:
            us = float(m["AverageNs"]) / 1e3
            gbs = multi_bytes(sizes) / (us * 1e-6) / 1e9
            lines += ["", f"compress_2bit_multi: {us:.2f} us per call = {gbs:,.0f} GB/s = "
                      f"{100 * gbs / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:,.0f} GB/s."]
        t = next((r for r in stats if r["Name"] == "compress_ternary_vec_kernel"), None)
        if t:
            us = float(t["AverageNs"]) / 1e3
            tb = 12 * n2 + 4 * ternary_words(n2)
            gbs = tb / (us * 1e-6) / 1e9
            lines += ["", f"compress_ternary at {n2:,} values: {tb:,} algorithmic bytes in "
                      f"{us:.2f} us = {gbs:,.0f} GB/s = {100 * gbs / HBM_PEAK_GBS:.1f}% of "
                      f"{HBM_PEAK_GBS:,.0f} GB/s."]
        lines += ["", f"kernel_source_sha256: {kernel_source_hash()}", ""]
        PROFILE_STATS_EXTRA.write_text("\n".join(lines))
        wrote.append(PROFILE_STATS_EXTRA)
    v = summarize_valu(d)
    if v:
        wrote.append(v)
    print("wrote " + ", ".join(str(w) for w in wrote))


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def calibrate_copy() -> None:
    import torch
    n = 1 << 28  # 1 GiB of fp32
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device copy", "bytes_read": 4 * n,
                      "bytes_written": 4 * n, "launches": 3}), flush=True)


def measure_ceilings(torch, steps: int) -> dict:
    """What this part's HBM gives each access mix of the hot path: the plain
    streaming kernels of libgcq_ceilings.so, which move exactly a hot-path
    kernel's bytes in its tile shapes with trivial arithmetic, timed with
    events around `steps` back-to-back launches that rotate over buffer sets
    (each mix's rotation is larger than the 256 MB Infinity Cache). Sizes
    are the workloads' rounded down to whole 16384-value quanta. For each
    mix: bytes per launch, ms per launch of every pattern (each also held to
    3, 4 and 5 resident workgroups per CU, "@k/CU"), the best one and its
    rate."""
    from gradient_compression_quantize_amd import ceilings as cl
    Q = cl.quantum()
    n2, n3 = N_C2 // Q * Q, N_C3 // Q * Q
    dev = "cuda"
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def zeros(count, dtype=torch.float32):
        return torch.zeros(count, dtype=dtype, device=dev)

    def timed(fns) -> float:
        for _ in range(2):
            for f in fns:
                f()
        torch.cuda.synchronize()
        a, b = mk(), mk()
        a.record()
        for k in range(steps):
            fns[k % len(fns)]()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def capped(patterns: dict) -> dict:
        """{pattern: launches} -> {pattern[@k/CU]: ms}, each pattern at
        every cap of CEILING_WG_PER_CU ("burst" runs 1024-thread workgroups
        with LDS of their own and is timed uncapped only)."""
        ms = {}
        for cap in CEILING_WG_PER_CU:
            cl.set_wg_per_cu(cap)
            for name, fns in patterns.items():
                if cap == 0:
                    ms[name] = timed(fns)
                elif name != "burst":
                    ms[f"{name}@{cap}/CU"] = timed(fns)
        cl.set_wg_per_cu(0)
        return ms

    def entry(nbytes, ms_by_pattern, n):
        best = min(ms_by_pattern, key=ms_by_pattern.get)
        gbs = nbytes / (ms_by_pattern[best] / 1e3) / 1e9
        return {"n": n, "bytes": nbytes, "ms": {k: round(v, 5) for k, v in ms_by_pattern.items()},
                "best": best, "gbs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}

    out = {"workloads": f"read and level sum at n = {n3:,} (VGG16 size, W = {W_C3}); write, "
                        f"compress and dequantize-sum at n = {n2:,} (ResNet-50 size, W = {W_C2})",
           "steps": steps}
    log("ceilings: read (the max-norm's stream)")
    bufs = [zeros(n3) for _ in range(W_C3)]
    sink = zeros(cl.read_sink_words(W_C3, n3), torch.int32)
    out["read"] = entry(4 * W_C3 * n3, capped({
        "chunked": [lambda: cl.read(bufs, n3, cl.READ_CHUNKED, sink)],
        "tile": [lambda: cl.read(bufs, n3, cl.READ_TILE, sink)]}), n3)
    del bufs, sink
    log("ceilings: level-sum mix")
    lv = [zeros(n3 // 4, torch.int32) for _ in range(W_C3)]
    sums, o3 = zeros(n3, torch.int32), zeros(n3)
    out["levelsum_mix"] = entry((W_C3 + 8) * n3,
                                capped({"tile": [lambda: cl.levelsum(lv, n3, sums, o3)]}), n3)
    del lv
    log("ceilings: fused quantize-sum mix")
    grads = [zeros(n3) for _ in range(W_C3)]
    out["quantize_sum_mix"] = entry((4 * W_C3 + 8) * n3, capped({
        "tile": [lambda: cl.quantize_sum(grads, n3, sums, o3)]}), n3)
    del grads, sums
    log("ceilings: quantize mix")
    src2, dst2 = [o3, zeros(n3)], [zeros(n3 // 4, torch.int32) for _ in range(2)]
    out["quantize_mix"] = entry(5 * n3, capped({"tile": [
        lambda k=k: cl.quantize(src2[k], n3, dst2[k]) for k in range(2)]}), n3)
    del src2, dst2, o3
    torch.cuda.empty_cache()
    log("ceilings: write")
    dsts = [zeros(n2) for _ in range(8)]
    out["write"] = entry(4 * n2, capped({
        "tile": [lambda d=d: cl.write(d, n2, cl.WRITE_TILE) for d in dsts],
        "stride": [lambda d=d: cl.write(d, n2, cl.WRITE_STRIDE) for d in dsts]}), n2)
    log("ceilings: compress mix")
    bw = cl.block_words(n2)
    sets = [(zeros(n2), zeros(n2), zeros(bw, torch.int32)) for _ in range(6)]
    out["compress_mix"] = entry(compress_bytes(n2), capped({"tile": [
        lambda st=st: cl.compress(st[0], st[1], n2, st[2]) for st in sets]}), n2)
    del sets
    log("ceilings: dequantize-sum mix")
    dsets = [[zeros(bw, torch.int32) for _ in range(W_C2)] for _ in range(8)]
    out["dequant_mix"] = entry(dequant_sum_bytes(n2, W_C2), capped({
        name: [lambda k=k, pat=pat: cl.dequant(dsets[k], n2, pat, dsts[k]) for k in range(8)]
        for name, pat in (("tile", cl.DEQ_TILE), ("wide", cl.DEQ_WIDE), ("burst", cl.DEQ_BURST))}),
        n2)
    log("ceilings: ternary dequantize-sum mix")
    nt = N_C2 // cl.ternary_quantum() * cl.ternary_quantum()
    tsets = [[zeros(3 + nt // 20, torch.int32) for _ in range(W_C2)] for _ in range(8)]
    out["dequant_ternary_mix"] = entry(4 * W_C2 * (3 + nt // 20) + 4 * nt, capped({
        "tile": [lambda k=k: cl.dequant_ternary(tsets[k], nt, dsts[k]) for k in range(8)]}),
        nt)
    del dsets, dsts, tsets
    torch.cuda.empty_cache()
    return out


def with_ceiling(roof: dict, gbs: float, ceil: dict | None, mix: str) -> dict:
    """Adds to a roofline object the kernel's rate over its access mix's
    measured ceiling (frac_of_ceiling) and that ceiling."""
    if ceil and mix in ceil:
        roof["ceiling"] = {"mix": mix, "gbs": ceil[mix]["gbs"], "pattern": ceil[mix]["best"]}
        roof["frac_of_ceiling"] = round(gbs / ceil[mix]["gbs"], 4)
    return roof


def bench_2bit(gcq, torch, np, si, steps: int, warmup: int):
    return bench_threshold_step(gcq, torch, si, steps, warmup, "2-bit",
                                gcq.gc_compressed_2bit_words, gcq.compress_2bit,
                                gcq.decompress_2bit_sum)


def bench_threshold_step(gcq, torch, si, steps: int, warmup: int, tag: str, words_of,
                         compress, dequant_sum):
    """W = 8 compresses (residual carried) + the W-block dequantize-sum at the
    ResNet-50 size, with one of the two packings of the threshold codes."""
    n, W = N_C2, W_C2
    dev = "cuda"
    log(f"{tag}: generating {W} x {n} fp32 gradients")
    grads = [torch.from_numpy(si.normal_f32(si.grad_seed(w, 0), n, SIGMA_C2)).to(dev)
             for w in range(W)]
    res = [torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(W)]
    words = words_of(n)
    comprs = [torch.empty(words, dtype=torch.int32, device=dev) for _ in range(W)]
    out = torch.empty(n, dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        for w in range(W):
            compress(grads[w], res[w], -THR_C2, THR_C2, comprs[w])
        if ev is not None:
            ev[1].record()
        dequant_sum(comprs, n, out)
        if ev is not None:
            ev[2].record()

    log(f"{tag}: warmup {warmup} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    # timed pass: K plain steps between two events
    t0, t1 = mk(), mk()
    log(f"{tag}: timing {steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t0.elapsed_time(t1) / steps
    # kernel pass: K more steps with events around the 8 back-to-back compress
    # launches and around the dequantize-sum; a compress launch's duration is
    # its group's time over 8 (events around every launch would add their own
    # packets' latency to each one)
    evs = [[mk() for _ in range(3)] for _ in range(steps)]
    log(f"{tag}: kernel timing over {steps} more steps")
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    comp_ms = [evs[k][0].elapsed_time(evs[k][1]) / W for k in range(steps)]
    deq_ms = [evs[k][1].elapsed_time(evs[k][2]) for k in range(steps)]
    # the dequantize-sum alone, timed like the ceiling kernels: K back-to-back
    # launches between two events, rotating over 8 copies of the step's
    # blocks and 8 outputs (1.2 GB, so the Infinity Cache cannot serve the
    # reads); one event pair around a single launch adds its own latency
    sets = [[c.clone() for c in comprs] for _ in range(8)]
    outs = [torch.empty_like(out) for _ in range(8)]
    for k in range(8):
        dequant_sum(sets[k], n, outs[k])
    torch.cuda.synchronize()
    d0, d1 = mk(), mk()
    d0.record()
    for k in range(steps):
        dequant_sum(sets[k % 8], n, outs[k % 8])
    d1.record()
    torch.cuda.synchronize()
    deq_b2b_ms = d0.elapsed_time(d1) / steps
    del sets, outs
    # the same step replayed from a HIP graph (no host launch cost)
    graph = graph_of(torch, step)
    g0, g1 = mk(), mk()
    g0.record()
    for _ in range(steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / steps
    del graph
    del grads, res, comprs, out
    torch.cuda.empty_cache()
    return {"ms_per_step": ms_step, "wall_s": wall, "compress_ms": comp_ms, "dequant_sum_ms": deq_ms,
            "dequant_sum_b2b_ms": deq_b2b_ms, "graph_ms_per_step": graph_ms}


def hbm_alu_roofline(name: str, kernel: str, nbytes: int, launch_s: float) -> dict:
    """Roofline of a kernel near both the HBM and the VALU-issue ceilings:
    algorithmic bytes over the live launch time against 8 TB/s, and (while
    the committed counter profile matches these sources) SQ_INSTS_VALU x 64
    lanes over the same time against the VALU peak. `bound` names the
    higher fraction."""
    gbs = nbytes / launch_s / 1e9
    r = {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
         "traffic": traffic_from_profile(kernel), "launch_ms": round(launch_s * 1e3, 5),
         "alu": None}
    vi = valu_insts_from_profile(kernel)
    if vi is not None:
        ach = vi * 64 / launch_s / 1e12
        r["alu"] = {"achieved": round(ach, 2), "peak": round(VALU_PEAK_T_LANE_INSTS, 2),
                    "unit": "T VALU lane-instructions/s",
                    "frac": round(ach / VALU_PEAK_T_LANE_INSTS, 4),
                    "valu_insts_per_launch": vi}
        if r["alu"]["frac"] > r["frac"]:
            r["bound"] = "alu"
    return r


def bench_qsgd(gcq, torch, np, si, steps: int):
    n, W, s = N_C3, W_C3, S_C3
    dev = "cuda"
    grads = []
    for w in range(W):
        log(f"qsgd: generating worker {w} ({n} heavy-tailed fp32)")
        grads.append(torch.from_numpy(si.heavy_tailed_f32(si.grad_seed(w, 0), n, SIGMA_C3)).to(dev))
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, n), dtype=torch.uint8, device=dev)
    levels = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(W)]
    sums = torch.empty(n, dtype=torch.int32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(seed, ev=None):
        if ev is not None:
            ev[0].record()
        gcq.qsgd_global_maxnorm(grads, norm, ws)
        if ev is not None:
            ev[1].record()
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(grads[w], norm, s, seed, w, levels[w])
        if ev is not None:
            ev[2].record()
        gcq.qsgd_dequant_sum(levels, norm, s, out, sums=sums)
        if ev is not None:
            ev[3].record()

    for _ in range(2):
        step(0)
    torch.cuda.synchronize()
    evs = [[mk() for _ in range(4)] for _ in range(steps)]
    log(f"qsgd: timing {steps} steps")
    for k in range(steps):
        step(0, evs[k])
    torch.cuda.synchronize()
    tot = [e[0].elapsed_time(e[3]) for e in evs]
    mx = [e[0].elapsed_time(e[1]) for e in evs]
    qz = [e[1].elapsed_time(e[2]) for e in evs]
    ds = [e[2].elapsed_time(e[3]) for e in evs]
    del levels

    # the same step with the W quantizes and the level sum fused (no int8
    # levels written): max-norm, then qsgd_quantize_sum
    def fused_step(seed, ev):
        ev[0].record()
        gcq.qsgd_global_maxnorm(grads, norm, ws)
        ev[1].record()
        gcq.qsgd_quantize_sum(grads, norm, s, seed, out, sums=sums)
        ev[2].record()

    fused_step(0, [mk() for _ in range(3)])
    torch.cuda.synchronize()
    fevs = [[mk() for _ in range(3)] for _ in range(steps)]
    log(f"qsgd: timing {steps} fused steps")
    for k in range(steps):
        fused_step(0, fevs[k])
    torch.cuda.synchronize()
    ftot = [e[0].elapsed_time(e[2]) for e in fevs]
    fqs = [e[1].elapsed_time(e[2]) for e in fevs]
    del grads, sums, out
    torch.cuda.empty_cache()
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    t = mean(tot) / 1e3
    # the quantize sits near two ceilings: HBM (4 B read + 1 B written per
    # value) and VALU issue (the Philox rounds). Its roofline gives both
    # fractions over the live per-launch time and names the higher one as
    # the bound. The max-norm's is HBM bytes.
    q_launch_s = mean(qz) / W / 1e3
    quant = hbm_alu_roofline("qsgd_quantize", "qsgd_quantize_kernel", 5 * n, q_launch_s)
    mx_gbs = 4 * W * n / (mean(mx) / 1e3) / 1e9
    hbm = {"bound": "hbm", "kernel": "qsgd_global_maxnorm", "achieved": round(mx_gbs, 1),
           "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(mx_gbs / HBM_PEAK_GBS, 4),
           "traffic": traffic_from_profile("maxabs_partial_kernel")}
    ls_gbs = (W + 8) * n / (mean(ds) / 1e3) / 1e9
    level_sum = {"bound": "hbm", "kernel": "qsgd_dequant_sum (dense level sum + dequantize)",
                 "achieved": round(ls_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ls_gbs / HBM_PEAK_GBS, 4),
                 "traffic": traffic_from_profile("qsgd_dequant_sum_kernel")}
    fused = {
        "workload": "the same step with qsgd_quantize_sum (W quantizes + level sum + dequantize "
                    "in one pass; the int8 levels are not written)",
        "ms_per_step": mean(ftot),
        "elems_per_s": W * n / (mean(ftot) / 1e3),
        "quantize_sum_ms": mean(fqs),
        "quantize_sum_gbs": (4 * W + 8) * n / (mean(fqs) / 1e3) / 1e9,
        "algorithmic_bytes": (4 * W + 4 * W + 8) * n,
        "roofline": hbm_alu_roofline("qsgd_quantize_sum", "qsgd_quantize_sum_kernel",
                                     (4 * W + 8) * n, mean(fqs) / 1e3),
    }
    return {
        "elems_per_s": W * n / t,
        "ms_per_step": mean(tot),
        "workload": f"QSGD-MN s={s}, {W} workers x {n} heavy-tailed fp32 (VGG16-sized): "
                    "global max-norm, quantize, int32 level sum, dequantize",
        "stages_ms": {"maxnorm": mean(mx), "quantize_x8": mean(qz), "dequant_sum": mean(ds)},
        "stages_gbs": {"maxnorm": 4 * W * n / (mean(mx) / 1e3) / 1e9,
                       "quantize_x8": 5 * W * n / (mean(qz) / 1e3) / 1e9,
                       "dequant_sum": (W + 8) * n / (mean(ds) / 1e3) / 1e9},
        "algorithmic_bytes": (4 * W + 5 * W + W + 8) * n,
        "steps": steps,
        "roofline": quant,
        "roofline_maxnorm": hbm,
        "roofline_level_sum": level_sum,
        "fused": fused,
    }


def graph_of(torch, fn):
    """Capture fn's launches (on torch's current stream) as a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def ternary_words(n: int) -> int:
    return 3 + (n + 19) // 20


def bench_ternary(gcq, torch, np, si, steps: int):
    """The 2-bit step's workload with the codes packed five per byte:
    compress_ternary x 8 workers + decompress_ternary_sum W = 8."""
    n, W = N_C2, W_C2
    r = bench_threshold_step(gcq, torch, si, steps, 3, "ternary", gcq.gc_compressed_ternary_words,
                             gcq.compress_ternary, gcq.decompress_ternary_sum)
    comp_b = 12 * n + 4 * ternary_words(n)
    deq_b = 4 * W * ternary_words(n) + 4 * n
    comp_ms = sum(r["compress_ms"]) / len(r["compress_ms"])
    deq_ms = r["dequant_sum_b2b_ms"]
    step_b = W * comp_b + deq_b
    comp_gbs = comp_b / (comp_ms / 1e3) / 1e9
    return {"workload": "dense ternary packing (5 codes per byte): compress_ternary x 8 workers "
                        f"({n:,} fp32 each, thresholds +-{THR_C2}, residual carried) + "
                        "decompress_ternary_sum W=8",
            "ms_per_step": r["ms_per_step"], "graph_ms_per_step": r["graph_ms_per_step"],
            "step_algorithmic_bytes": step_b,
            "gbs": step_b / (r["ms_per_step"] / 1e3) / 1e9,
            "compress_ternary": {"avg_ms": comp_ms, "algorithmic_bytes": comp_b,
                                 "gbs": comp_gbs},
            "decompress_ternary_sum": {"avg_ms": deq_ms, "algorithmic_bytes": deq_b,
                                       "gbs": deq_b / (deq_ms / 1e3) / 1e9,
                                       "frac": round(deq_b / (deq_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                       "timing": "back-to-back launches over 8 rotating block sets",
                                       "in_step_avg_ms": sum(r["dequant_sum_ms"]) / len(r["dequant_sum_ms"])},
            "roofline": {"bound": "hbm", "kernel": "compress_ternary",
                         "achieved": round(comp_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_from_profile("compress_ternary_vec_kernel")},
            "wire_bytes_per_worker": 4 * ternary_words(n),
            "wire_bytes_per_worker_2bit": 4 * (3 + (n + 15) // 16),
            "oracle_ms": None, "steps": steps}


def bench_many_workers(gcq, torch, steps: int):
    """The W-block dequantize-sums at the ResNet-50 size for W above the
    compile-time range (16 and 64 workers: the run-time-W kernels), on
    random-bit blocks with thresholds +-0.5, rotating over block sets of at
    least 1 GB."""
    n = N_C2
    out = {"workload": f"decompress_2bit_sum and decompress_ternary_sum, n = {n:,}, random "
                       "payload bits, W = 16 and 64",
           "steps": steps}
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for tag, words_of, fn in (("2bit", gcq.gc_compressed_2bit_words, gcq.decompress_2bit_sum),
                              ("ternary", gcq.gc_compressed_ternary_words,
                               gcq.decompress_ternary_sum)):
        for W in (16, 64):
            log(f"many workers: {tag} W={W}")
            nw = words_of(n)
            R = max(2, -(-(1 << 30) // (W * nw * 4)))
            gen = torch.Generator(device="cuda")
            gen.manual_seed(7 * W)
            sets = []
            for _ in range(R):
                bl = []
                for _ in range(W):
                    b = torch.randint(-2 ** 31, 2 ** 31 - 1, (nw,), dtype=torch.int32,
                                      device="cuda", generator=gen)
                    b[0], b[1], b[2] = -0x41000000, 0x3F000000, 0  # -0.5, 0.5 as fp32 bits
                    bl.append(b)
                sets.append(bl)
            dst = [torch.empty(n, device="cuda") for _ in range(2)]
            for r in range(R):
                fn(sets[r], n, dst[r % 2])
            torch.cuda.synchronize()
            reps = max(steps, 2 * R)
            a, b = mk(), mk()
            a.record()
            for k in range(reps):
                fn(sets[k % R], n, dst[k % 2])
            b.record()
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / reps
            nbytes = W * 4 * nw + 4 * n
            out[f"{tag}_w{W}"] = {"ms": round(ms, 5), "bytes": nbytes,
                                  "gbs": round(nbytes / (ms / 1e3) / 1e9, 1)}
            del sets, dst
            torch.cuda.empty_cache()
    return out


def bench_misaligned(gcq, torch, si, steps: int):
    """The 2-bit and ternary kernels on buffers 4 bytes off 16-byte alignment
    (views at element offset 1, as inside a flat bucket of odd-sized
    tensors), beside the same calls on aligned buffers: compress of one
    ResNet-50-sized worker and the W = 8 dequantize-sum."""
    n, W = N_C2, W_C2
    dev = "cuda:0"
    grads = []
    for w in range(W):
        g = si.uniform_f32_device(7000 + w, n + 1, dev)
        g.mul_(2 * SIGMA_C2)
        grads.append(g)
    res = torch.zeros(n + 1, dtype=torch.float32, device=dev)
    out = torch.empty(n + 1, dtype=torch.float32, device=dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def per_call(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    result = {"workload": f"compress of one worker and the W={W} dequantize-sum, n={n:,}, on "
                          "buffers 4 bytes off 16-byte alignment (element offset 1) and on "
                          "aligned buffers", "steps": steps}
    for name, words, comp, dsum in (("2bit", gcq.gc_compressed_2bit_words, gcq.compress_2bit,
                                     gcq.decompress_2bit_sum),
                                    ("ternary", gcq.gc_compressed_ternary_words,
                                     gcq.compress_ternary, gcq.decompress_ternary_sum)):
        blocks = [torch.empty(words(n), dtype=torch.int32, device=dev) for _ in range(W)]
        comp_b = 12 * n + 4 * words(n)
        deq_b = 4 * W * words(n) + 4 * n
        entry = {}
        for off, key in ((1, "misaligned"), (0, "aligned")):
            views = [g[off:off + n] for g in grads]
            r, o = res[off:off + n], out[off:off + n]
            for w in range(W):
                comp(views[w], r, -THR_C2, THR_C2, blocks[w])
            c_ms = per_call(lambda: comp(views[0], r, -THR_C2, THR_C2, blocks[0]))
            d_ms = per_call(lambda: dsum(blocks, n, o))
            entry[key] = {"compress_ms": round(c_ms, 5),
                          "compress_gbs": round(comp_b / (c_ms / 1e3) / 1e9, 1),
                          "dequant_sum_ms": round(d_ms, 5),
                          "dequant_sum_gbs": round(deq_b / (d_ms / 1e3) / 1e9, 1)}
        result[name] = entry
        del blocks
    del grads, res, out
    torch.cuda.empty_cache()
    # QSGD-MN at the VGG16 size: max-norm over the W workers, one worker's
    # quantize, the W-level sum, and the fused quantize-sum
    nq, s, seed = N_C3, S_C3, 0
    qgrads = []
    for w in range(W):
        g = si.uniform_f32_device(7100 + w, nq + 1, dev)
        g.mul_(2 * SIGMA_C3)
        qgrads.append(g)
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    ws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, nq), dtype=torch.uint8, device=dev)
    lv_buf = [torch.empty(nq + 4, dtype=torch.int8, device=dev) for _ in range(W)]
    sums_buf = torch.empty(nq + 1, dtype=torch.int32, device=dev)
    out_buf = torch.empty(nq + 1, dtype=torch.float32, device=dev)
    qsteps = max(2, steps // 4)
    entry = {"workload": f"QSGD-MN, s={s}, W={W} x {nq:,} values; misaligned: gradients, sums "
                         "and outputs at element offset 1, levels at byte offset 4; "
                         "levels_at_byte_offsets: worker w's int8 levels at byte offset "
                         "1 + w % 3, everything else aligned"}
    for off, key in ((1, "misaligned"), (0, "aligned")):
        gv = [g[off:off + nq] for g in qgrads]
        lv = [b[4 * off:4 * off + nq] for b in lv_buf]
        sm, o = sums_buf[off:off + nq], out_buf[off:off + nq]
        gcq.qsgd_global_maxnorm(gv, norm, ws)
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(gv[w], norm, s, seed, w, lv[w])
        entry[key] = {
            "maxnorm_ms": round(per_call(lambda: gcq.qsgd_global_maxnorm(gv, norm, ws)), 5),
            "quantize_one_worker_ms": round(per_call(
                lambda: gcq.qsgd_maxnorm_quantize(gv[0], norm, s, seed, 0, lv[0])), 5),
            "dequant_sum_ms": round(per_call(lambda: gcq.qsgd_dequant_sum(lv, norm, s, o, sums=sm)), 5),
        }
        for _ in range(2):
            gcq.qsgd_quantize_sum(gv, norm, s, seed, o, sums=sm)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(qsteps):
            gcq.qsgd_quantize_sum(gv, norm, s, seed, o, sums=sm)
        b.record()
        torch.cuda.synchronize()
        entry[key]["quantize_sum_ms"] = round(a.elapsed_time(b) / qsteps, 5)
    # int8 levels 1-3 bytes past a 4-byte boundary (worker w at 1 + w % 3),
    # the gradients and outputs aligned: the quantize and the level sum
    gv = [g[0:nq] for g in qgrads]
    lv = [b[1 + w % 3:1 + w % 3 + nq] for w, b in enumerate(lv_buf)]
    sm, o = sums_buf[0:nq], out_buf[0:nq]
    gcq.qsgd_global_maxnorm(gv, norm, ws)
    for w in range(W):
        gcq.qsgd_maxnorm_quantize(gv[w], norm, s, seed, w, lv[w])
    entry["levels_at_byte_offsets"] = {
        "quantize_one_worker_ms": round(per_call(
            lambda: gcq.qsgd_maxnorm_quantize(gv[1], norm, s, seed, 1, lv[1])), 5),
        "dequant_sum_ms": round(per_call(lambda: gcq.qsgd_dequant_sum(lv, norm, s, o, sums=sm)), 5),
    }
    al = entry["aligned"]
    entry["levels_at_byte_offsets"]["vs_aligned"] = {
        "quantize": round(entry["levels_at_byte_offsets"]["quantize_one_worker_ms"]
                          / al["quantize_one_worker_ms"], 3),
        "dequant_sum": round(entry["levels_at_byte_offsets"]["dequant_sum_ms"]
                             / al["dequant_sum_ms"], 3)}
    result["qsgd"] = entry
    del qgrads, lv_buf, sums_buf, out_buf, ws
    torch.cuda.empty_cache()
    return result


def multi_bytes(sizes) -> int:
    return sum(12 * n + 4 * (3 + (n + 15) // 16) for n in sizes)


def bench_multi(gcq, torch, np, si, steps: int):
    """Many-tensor 2-bit compress over the BERT-Base parameter list (198
    tensors, 109,482,240 values, thresholds +-0.005): one launch per step."""
    sizes = si.bert_base_sizes()
    dev = "cuda"
    log(f"multi-tensor: generating {len(sizes)} tensors ({sum(sizes)} values)")
    host = [si.normal_f32(7919 * t, n, 0.005) for t, n in enumerate(sizes)]
    grads = [torch.from_numpy(h).to(dev) for h in host]
    res = [torch.zeros(n, dtype=torch.float32, device=dev) for n in sizes]
    plan = gcq.Plan2bitMulti(grads, res)
    compr = torch.empty(plan.compressed_words, dtype=torch.int32, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for _ in range(3):
        plan.compress(-0.005, 0.005, compr)
    torch.cuda.synchronize()
    t0, t1 = mk(), mk()
    t0.record()
    for _ in range(steps):
        plan.compress(-0.005, 0.005, compr)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    plan.destroy()
    del grads, res, compr
    torch.cuda.empty_cache()
    byts = multi_bytes(sizes)
    gbs = byts / (ms / 1e3) / 1e9
    del host
    return {"workload": "compress_2bit_multi over the BERT-Base parameter list: 198 tensors, "
                        f"{sum(sizes):,} fp32 values, thresholds +-0.005, one launch",
            "ms_per_call": ms, "algorithmic_bytes": byts, "gbs": gbs,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4)},
            "oracle_ms_per_call": None, "steps": steps}


def bench_grandk(gcq, torch, np, si, steps: int):
    """GlobalRandK-MN at the ResNet-50 size: shared K = 10000 indices, gather
    for 8 workers, max-norm, quantize at s = 7, level sum and scatter into a
    dense fp32 buffer (the dense zero fill dominates the bytes)."""
    n, K, W, s = N_C2, 10_000, W_C2, 7
    dev = "cuda"
    log("grandk: generating inputs")
    host = [si.normal_f32(si.grad_seed(w, 0), n, SIGMA_C2) for w in range(W)]
    grads = [torch.from_numpy(h).to(dev) for h in host]
    idx = torch.empty(K, dtype=torch.int32, device=dev)
    ws = torch.empty(gcq.grandk_ws_bytes(n, K), dtype=torch.uint8, device=dev)
    gathered = [torch.empty(K, dtype=torch.float32, device=dev) for _ in range(W)]
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    mws = torch.empty(gcq.qsgd_maxnorm_ws_bytes(W, K), dtype=torch.uint8, device=dev)
    levels = [torch.empty(K, dtype=torch.int8, device=dev) for _ in range(W)]
    sums = torch.empty(K, dtype=torch.int32, device=dev)
    dense = torch.empty(n, dtype=torch.float32, device=dev)
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(seed, ev=None):
        if ev is not None:
            ev[0].record()
        gcq.grandk_indices(n, K, seed, idx, ws)
        if ev is not None:
            ev[1].record()
        for w in range(W):
            gcq.gather_f32(grads[w], idx, gathered[w])
        gcq.qsgd_global_maxnorm(gathered, norm, mws)
        for w in range(W):
            gcq.qsgd_maxnorm_quantize(gathered[w], norm, s, seed, w, levels[w])
        if ev is not None:
            ev[2].record()
        gcq.qsgd_dequant_sum(levels, norm, s, dense, sums=sums, scatter_idx=idx, dense_n=n)
        if ev is not None:
            ev[3].record()

    for k in range(3):
        step(k)
    torch.cuda.synchronize()
    # eager pass with events between the stages
    evs = [[mk() for _ in range(4)] for _ in range(steps)]
    for k in range(steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    mean = lambda v: sum(v) / len(v)  # noqa: E731
    eager = mean([e[0].elapsed_time(e[3]) for e in evs])
    draw = mean([e[0].elapsed_time(e[1]) for e in evs])
    mid = mean([e[1].elapsed_time(e[2]) for e in evs])
    fill = mean([e[2].elapsed_time(e[3]) for e in evs])
    # the step's 20 small launches captured once as a HIP graph and replayed
    graph = graph_of(torch, lambda: step(0))
    t0, t1 = mk(), mk()
    t0.record()
    for _ in range(steps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    sep_graph = t0.elapsed_time(t1) / steps
    del graph

    # the same step through grandk_mn_step: three launches
    sws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, n, K), dtype=torch.uint8, device=dev)

    def one_call(seed):
        gcq.grandk_mn_step(grads, K, seed, s, idx, dense, sws, sums=sums, norm=norm)

    gpu_ms, eager_ms, host_us = time_grandk_calls(torch, one_call, steps)
    # the latency chain alone: the same step on n = 2^20 values, whose fill
    # is ~0.7 us
    nc = 1 << 20
    cgrads = [g[:nc] for g in grads]
    cdense = torch.empty(nc, dtype=torch.float32, device=dev)
    cws = torch.empty(gcq.grandk_mn_step_ws_bytes(W, nc, K), dtype=torch.uint8, device=dev)
    chain_ms, _, _ = time_grandk_calls(
        torch, lambda seed: gcq.grandk_mn_step(cgrads, K, seed, s, idx, cdense, cws, sums=sums,
                                               norm=norm), steps)
    del grads, dense, sws, cgrads, cdense, cws
    torch.cuda.empty_cache()
    del host
    dense_gbs = 4 * n / (fill / 1e3) / 1e9
    step_gbs = 4 * n / (gpu_ms / 1e3) / 1e9
    return {"workload": f"GRandK-MN: n={n:,}, K={K}, W={W}, s={s}: shared index draw, gather, "
                        "max-norm, quantize, level sum, scatter into a dense fp32 buffer",
            "ms_per_step": gpu_ms, "values_per_s": K * W / (gpu_ms / 1e3),
            "timing": f"grandk_mn_step (three launches): a HIP graph of {GK_GRAPH_STEPS} steps "
                      "replayed back to back, so the GPU never waits for the host",
            "eager_ms_per_step": eager_ms,
            "host_us_per_call": round(host_us, 2),
            "eager_timing": "the same calls issued one by one from Python between two events; "
                            "host_us_per_call is the binding's host time per call (argument "
                            "checks, marshalling, three kernel launches): where it exceeds the "
                            "GPU's time, eager_ms_per_step measures the host",
            "chain_ms_per_step": chain_ms,
            "chain_timing": f"the same step at n = {nc:,} (a 4 MB fill), graph-timed: the "
                            "draw -> gather -> norm -> quantize -> scatter chain and its launch "
                            "gaps without the bulk of the fill",
            "separate_calls": {
                "timing": "the 20 separate calls (draw, W gathers, max-norm, W quantizes, "
                          "dequantize-scatter): HIP graph replay; stages from an eager pass",
                "ms_per_step": sep_graph, "ms_per_step_eager": eager,
                "stages_ms": {"index_draw": draw, "gather_norm_quantize": mid,
                              "sum_fill_scatter": fill},
                "fill_scatter_gbs": round(dense_gbs, 1)},
            # the dense output (4 n bytes, zeroed and scattered once) dominates
            # the step's bytes; the rest is under 1 MB
            "roofline": {"bound": "hbm",
                         "kernel": "grandk_mn_step, whole step (dense output written once)",
                         "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                         "traffic": traffic_from_profile("grandk_mn_step", PROFILE_GRANDK,
                                                         "traffic_bytes_per_step")},
            "oracle_ms_per_step": None, "steps": steps}


GK_GRAPH_STEPS = 20


def time_grandk_calls(torch, call, steps: int):
    """(GPU ms per step, eager ms per step, host us per call) of call(seed):
    the GPU time from a HIP graph of GK_GRAPH_STEPS calls replayed back to
    back; the eager time from `steps` calls issued one by one; the host time
    from the wall clock around those calls."""
    mk = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for k in range(3):
        call(k)
    torch.cuda.synchronize()
    t0, t1 = mk(), mk()
    h0 = time.perf_counter()
    t0.record()
    for k in range(steps):
        call(k)
    h1 = time.perf_counter()
    t1.record()
    torch.cuda.synchronize()
    eager = t0.elapsed_time(t1) / steps
    host_us = (h1 - h0) / steps * 1e6

    def many():
        for k in range(GK_GRAPH_STEPS):
            call(k)

    graph = graph_of(torch, many)
    reps = max(3, steps // GK_GRAPH_STEPS)
    graph.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    gpu = t0.elapsed_time(t1) / (reps * GK_GRAPH_STEPS)
    del graph
    return gpu, eager, host_us


def cpu_baseline(np, si, budget_s: float, workloads=()):
    """The oracle, untouched, on the same 2-bit step (8 workers' compress +
    the W = 8 dequantize-sum), repeated until the time budget is spent; then,
    for each other workload the run measured (`workloads`), the oracle once
    on that workload or a stated sample of it. Single-threaded, pinned to
    one host core."""
    import oracle
    n, W = N_C2, W_C2
    log("cpu baseline: generating inputs")
    grads = [si.normal_f32(si.grad_seed(w, 0), n, SIGMA_C2) for w in range(W)]
    res = [np.zeros(n, np.float32) for _ in range(W)]
    gq = None
    if "qsgd" in workloads:
        # the whole VGG16-sized workload, drawn before the process is pinned
        # to one core (one thread per worker; not timed)
        from concurrent.futures import ThreadPoolExecutor
        log(f"cpu baseline: generating the QSGD-MN inputs ({W_C3} x {N_C3})")
        with ThreadPoolExecutor(max(1, min(W_C3, os.cpu_count() or 1))) as ex:
            gq = list(ex.map(lambda w: si.heavy_tailed_f32(si.grad_seed(w, 0), N_C3, SIGMA_C3),
                             range(W_C3)))
    oracle.lib()
    per = {}
    # one core for the timed loop (the oracle is single-threaded); restored after
    saved = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    pinned = None
    if saved:
        pinned = min(saved)
        os.sched_setaffinity(0, {pinned})
    try:
        reps = 0
        t0 = time.perf_counter()
        while True:
            blocks = [oracle.quantize_2bit(grads[w], res[w], -THR_C2, THR_C2) for w in range(W)]
            oracle.dequantize_2bit_sum(blocks, n)
            reps += 1
            el = time.perf_counter() - t0
            log(f"cpu baseline: step {reps} done ({el:.1f} s)")
            if el >= budget_s:
                break
        del blocks, res
        if "ternary" in workloads:
            # one worker's compress and the W-block sum
            c0 = time.perf_counter()
            blk = oracle.quantize_ternary(grads[0], np.zeros(n, np.float32), -THR_C2, THR_C2)
            comp_ms = (time.perf_counter() - c0) * 1e3
            c0 = time.perf_counter()
            oracle.dequantize_ternary_sum([blk] * W, n)
            per["ternary"] = {"compress_one_worker": comp_ms,
                              "dequant_sum_w8": (time.perf_counter() - c0) * 1e3}
            log("cpu baseline: ternary done")
        if "grandk" in workloads:
            # the whole GRandK-MN step at K = 10000 on the same 8 gradients
            K, s = 10_000, 7
            c0 = time.perf_counter()
            idx_h = oracle.randk_indices(n, K, 0)
            gk = [oracle.gather(g, idx_h) for g in grads]
            nrm = oracle.maxnorm(gk)
            lv = [oracle.qsgd_quantize(gk[w], nrm, s, 0, w) for w in range(W)]
            oracle.scatter_dense(oracle.qsgd_dequantize(oracle.level_sum(lv), nrm, s), idx_h, n)
            per["grandk"] = (time.perf_counter() - c0) * 1e3
            log("cpu baseline: grandk done")
        del grads
        if "multi" in workloads:
            # one pass over the BERT-Base tensor list
            sizes = si.bert_base_sizes()
            host = [si.normal_f32(7919 * t, m, 0.005) for t, m in enumerate(sizes)]
            res_h = [np.zeros(m, np.float32) for m in sizes]
            c0 = time.perf_counter()
            for t in range(len(sizes)):
                oracle.quantize_2bit(host[t], res_h[t], -0.005, 0.005)
            per["multi"] = (time.perf_counter() - c0) * 1e3
            del host, res_h
            log("cpu baseline: multi-tensor done")
        if "qsgd" in workloads:
            # the whole QSGD-MN step (max-norm, W quantizes, level sum,
            # dequantize) on the full workload: about 15 s on one core
            Wq, sq = W_C3, S_C3
            c0 = time.perf_counter()
            nrm = oracle.maxnorm(gq)
            lv = [oracle.qsgd_quantize(gq[w], nrm, sq, 0, w) for w in range(Wq)]
            oracle.qsgd_dequantize(oracle.level_sum(lv), nrm, sq)
            el_q = time.perf_counter() - c0
            del lv
            per["qsgd"] = {"sample": f"the whole step on {Wq} workers x {N_C3:,} heavy-tailed "
                                     "values (the full workload)",
                           "ms": el_q * 1e3,
                           "values_per_s": Wq * N_C3 / el_q}
            log(f"cpu baseline: qsgd step done ({el_q:.1f} s)")
        del gq
    finally:
        if saved:
            os.sched_setaffinity(0, saved)
    step_s = el / reps
    gbs = (W * compress_bytes(n) + dequant_sum_bytes(n, W)) / step_s / 1e9
    return {"value": gbs, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full 2-bit steps (8 x {n} values compressed + W=8 dequantize-sum) "
                      f"in {el:.1f} s, single-threaded C oracle pinned to host core {pinned} "
                      f"({cpu_model()}, {os.cpu_count()} visible)",
            "values_per_s": W * n / step_s,
            "ms_per_step": step_s * 1e3,
            "per_workload": per}


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this library runs on one GPU; multi-GPU runs are not part of it "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return 0
    import numpy as np
    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return 0
    if args.calibrate_ceilings:
        if not torch.cuda.is_available():
            print("bench.py: no GPU visible", file=sys.stderr)
            return 1
        print(json.dumps({"hbm_ceilings": measure_ceilings(torch, args.ceiling_steps)}), flush=True)
        return 0

    import gradient_compression_quantize_amd as gcq
    import synthetic_inputs as si

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    gcq.load()
    if args.extras_only:
        print(json.dumps({"multi_tensor": bench_multi(gcq, torch, np, si, args.extra_steps),
                          "grandk_mn": bench_grandk(gcq, torch, np, si, args.extra_steps),
                          "ternary": bench_ternary(gcq, torch, np, si, args.extra_steps),
                          "misaligned": bench_misaligned(gcq, torch, si, args.extra_steps),
                          "many_workers": bench_many_workers(gcq, torch, args.extra_steps)}),
              flush=True)
        return 0

    r2 = bench_2bit(gcq, torch, np, si, args.steps, args.warmup)
    step_bytes = W_C2 * compress_bytes(N_C2) + dequant_sum_bytes(N_C2, W_C2)
    ms = r2["ms_per_step"]
    value = step_bytes / (ms / 1e3) / 1e9
    comp_ms = sum(r2["compress_ms"]) / len(r2["compress_ms"])
    deq_ms = sum(r2["dequant_sum_ms"]) / len(r2["dequant_sum_ms"])
    comp_gbs = compress_bytes(N_C2) / (comp_ms / 1e3) / 1e9
    deq_b2b_ms = r2["dequant_sum_b2b_ms"]
    deq_gbs = dequant_sum_bytes(N_C2, W_C2) / (deq_b2b_ms / 1e3) / 1e9
    traffic = traffic_from_profile("compress_2bit_vec_kernel")

    result = {
        "metric": "2-bit EF quantize+pack GB/s and % HBM peak, 25.6M fp32; QSGD-MN elems/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "graph_ms_per_step": round(r2["graph_ms_per_step"], 5),
        "config": {
            "workload": "2-bit EF step: compress_2bit x 8 workers (25,557,032 fp32 each, "
                        "ResNet-50-sized flat gradient, thresholds +-0.01, residual carried) "
                        "+ decompress_2bit_sum W=8",
            "n": N_C2, "workers": W_C2, "neg_threshold": -THR_C2, "pos_threshold": THR_C2,
            "sigma": SIGMA_C2, "step_algorithmic_bytes": step_bytes,
        },
        "kernels": {
            "compress_2bit": {"avg_ms": round(comp_ms, 5),
                              "median_ms": round(statistics.median(r2["compress_ms"]), 5),
                              "min_ms": round(min(r2["compress_ms"]), 5),
                              "gbs": round(comp_gbs, 1),
                              "algorithmic_bytes": compress_bytes(N_C2),
                              "launches": W_C2 * len(r2["compress_ms"]),
                              "timing": "per step, the 8 back-to-back launches between two "
                                        "events, divided by 8"},
            "decompress_2bit_sum": {"avg_ms": round(deq_b2b_ms, 5),
                                    "gbs": round(deq_gbs, 1),
                                    "frac": round(deq_gbs / HBM_PEAK_GBS, 4),
                                    "timing": f"{args.steps} back-to-back launches between two "
                                              "events over 8 rotating block sets",
                                    "in_step_avg_ms": round(deq_ms, 5),
                                    "in_step_median_ms": round(statistics.median(r2["dequant_sum_ms"]), 5),
                                    "in_step_timing": "one event pair around the launch in each step",
                                    "algorithmic_bytes": dequant_sum_bytes(N_C2, W_C2),
                                    "launches": len(r2["dequant_sum_ms"]) + args.steps},
        },
        "roofline": {"bound": "hbm", "kernel": "compress_2bit",
                     "achieved": round(comp_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }

    if not args.skip_qsgd:
        q = bench_qsgd(gcq, torch, np, si, args.qsgd_steps)
        result["qsgd_mn_elems_per_s"] = q["elems_per_s"]
        result["qsgd_mn"] = q
    if not args.skip_extra:
        result["multi_tensor"] = bench_multi(gcq, torch, np, si, args.extra_steps)
        result["grandk_mn"] = bench_grandk(gcq, torch, np, si, args.extra_steps)
        result["ternary"] = bench_ternary(gcq, torch, np, si, args.extra_steps)
        result["misaligned"] = bench_misaligned(gcq, torch, si, args.extra_steps)
        result["many_workers"] = bench_many_workers(gcq, torch, args.extra_steps)

    if not args.skip_ceilings:
        ceil = measure_ceilings(torch, args.ceiling_steps)
        result["hbm_ceilings"] = ceil
        with_ceiling(result["roofline"], comp_gbs, ceil, "compress_mix")
        dk = result["kernels"]["decompress_2bit_sum"]
        with_ceiling(dk, dk["gbs"], ceil, "dequant_mix")
        if "qsgd_mn" in result:
            q = result["qsgd_mn"]
            with_ceiling(q["roofline"], q["roofline"]["achieved"], ceil, "quantize_mix")
            with_ceiling(q["roofline_maxnorm"], q["roofline_maxnorm"]["achieved"], ceil, "read")
            with_ceiling(q["roofline_level_sum"], q["roofline_level_sum"]["achieved"], ceil,
                         "levelsum_mix")
            if "fused" in q:
                with_ceiling(q["fused"]["roofline"], q["fused"]["roofline"]["achieved"], ceil,
                             "quantize_sum_mix")
        if "multi_tensor" in result:
            m = result["multi_tensor"]
            with_ceiling(m["roofline"], m["gbs"], ceil, "compress_mix")
        if "ternary" in result:
            t = result["ternary"]
            with_ceiling(t["roofline"], t["compress_ternary"]["gbs"], ceil, "compress_mix")
            td = t["decompress_ternary_sum"]
            with_ceiling(td, td["gbs"], ceil, "dequant_ternary_mix")
        if "grandk_mn" in result:
            g = result["grandk_mn"]
            with_ceiling(g["roofline"], g["roofline"]["achieved"], ceil, "write")

    if not args.skip_cpu_baseline:
        workloads = set()
        if not args.skip_qsgd:
            workloads.add("qsgd")
        if not args.skip_extra:
            workloads |= {"multi", "grandk", "ternary"}
        cb = cpu_baseline(np, si, args.cpu_seconds, workloads)
        result["cpu_baseline"] = cb
        # each workload's object also carries the oracle's time beside its own
        per = cb["per_workload"]
        if "qsgd" in per:
            result["qsgd_mn"]["oracle"] = dict(per["qsgd"], cores=1)
        if "multi" in per:
            result["multi_tensor"].update(oracle_ms_per_call=per["multi"], oracle_cores=1)
        if "grandk" in per:
            result["grandk_mn"].update(oracle_ms_per_step=per["grandk"], oracle_cores=1)
        if "ternary" in per:
            result["ternary"].update(oracle_ms=per["ternary"], oracle_cores=1)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
