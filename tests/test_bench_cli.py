"""bench.py's command-line contract, on the CPU: more than one GPU is
refused with a message (this library runs on one GPU), and a run with no
GPU visible fails with a message instead of printing a result line. Also
the rule that names a kernel's roofline bound, and the profile summaries
read from synthetic rocprofv3 CSV files."""
import json
import os
import pathlib
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent


def run(*args, env=None):
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = run(env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_no_gpu_no_result_line():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = run("--steps", "1", "--warmup", "0", env=env)
    assert r.returncode != 0
    for line in r.stdout.splitlines():
        try:
            obj = json.loads(line)
        except ValueError:
            continue
        assert "value" not in obj


def test_roofline_names_the_higher_fraction(monkeypatch):
    """A kernel near both ceilings reports its HBM and VALU fractions over
    the same launch time and is called bound by the higher one; without a
    profile taken on these sources the VALU half is absent."""
    sys.path.insert(0, str(ROOT))
    import bench
    monkeypatch.setattr(bench, "traffic_from_profile", lambda k: None)
    monkeypatch.setattr(bench, "valu_insts_from_profile", lambda k: None)
    r = bench.hbm_alu_roofline("k", "k_kernel", 4_000_000_000, 1e-3)  # 4 TB/s
    assert r["bound"] == "hbm" and r["alu"] is None and abs(r["frac"] - 0.5) < 1e-9
    # 0.8 of the VALU peak over 1 ms: more than the HBM half
    insts = int(0.8 * bench.VALU_PEAK_T_LANE_INSTS * 1e12 * 1e-3 / 64)
    monkeypatch.setattr(bench, "valu_insts_from_profile", lambda k: insts)
    r = bench.hbm_alu_roofline("k", "k_kernel", 4_000_000_000, 1e-3)
    assert r["bound"] == "alu" and abs(r["alu"]["frac"] - 0.8) < 1e-3
    # 0.3 of it: HBM stays the bound
    insts = int(0.3 * bench.VALU_PEAK_T_LANE_INSTS * 1e12 * 1e-3 / 64)
    monkeypatch.setattr(bench, "valu_insts_from_profile", lambda k: insts)
    assert bench.hbm_alu_roofline("k", "k_kernel", 4_000_000_000, 1e-3)["bound"] == "hbm"


def _write_trace(path: pathlib.Path, rows) -> None:
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    fields = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X",
              "Workgroup_Size_X", "LDS_Block_Size"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for name, start, end, grid in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": start, "End_Timestamp": end,
                        "Grid_Size_X": grid, "Workgroup_Size_X": 256, "LDS_Block_Size": 0})


def test_grandk_critical_path_summary_from_a_trace(tmp_path, monkeypatch):
    """The GlobalRandK summary finds the step's three launches in a kernel
    trace, tells the full-size steps from the n = 2^20 ones by launch 1's
    grid, and reports each launch's median duration and the gaps (ns
    timestamps in, us out)."""
    sys.path.insert(0, str(ROOT))
    import bench
    rows, t = [], 0

    def step(grid, d1, d2, d3, gap):
        nonlocal t
        for name, d, g in (("grandk_draw_fill_kernel", d1, grid),
                           ("grandk_gather_fill_kernel", d2, 9000),
                           ("grandk_quantize_scatter_kernel", d3, 8000)):
            rows.append((name, t, t + d, g))
            t += d + gap

    for _ in range(3):
        step(1_188_864, 14_000, 8_000, 4_500, 1_000)
    for _ in range(3):
        step(64_512, 12_500, 4_500, 4_500, 2_000)
    rows.append(("fill_zero_kernel", t, t + 17_800, 4096))
    _write_trace(tmp_path / "prof_extra" / "extra_kernel_trace.csv", rows)
    out = tmp_path / "gk.md"
    monkeypatch.setattr(bench, "PROFILE_GRANDK", out)
    monkeypatch.setattr(bench, "PROFILE_CEILINGS", tmp_path / "no_ceilings.md")
    assert bench.summarize_grandk_path(tmp_path) == out
    text = out.read_text()
    assert "| 14.00 | 12.50 |" in text  # launch 1, full size | n = 2^20
    assert "| 8.00 | 4.50 |" in text    # launch 2
    assert "| 1.00 | 2.00 |" in text    # gaps
    assert "| 28.50 | 25.50 |" in text  # first start to last end
    assert "17.80" in text              # the fill run alone


def test_grandk_summary_needs_the_trace(tmp_path):
    sys.path.insert(0, str(ROOT))
    import bench
    assert bench.summarize_grandk_path(tmp_path) is None


def test_ceiling_summary_splits_each_kernel_by_cap(tmp_path, monkeypatch):
    """measure_ceilings times each pattern once per cap, in the order of
    CEILING_WG_PER_CU, with equal launch counts: the summary assigns a
    kernel's launches in time order to the caps in equal runs, and the burst
    pattern (uncapped only) to one run."""
    sys.path.insert(0, str(ROOT))
    import bench
    rows, t = [], 0
    caps = bench.CEILING_WG_PER_CU
    for i, _ in enumerate(caps):
        for _ in range(4):  # 4 launches per cap, 10, 20, 30, ... us
            rows.append(("ceil_compress_mix_kernel", t, t + 10_000 * (i + 1), 6240))
            t += 100_000
    rows.append(("ceil_dequant_burst_kernel", t, t + 7_000, 1560))
    _write_trace(tmp_path / "prof_ceilings" / "ceil_kernel_trace.csv", rows)
    out = tmp_path / "ceil.md"
    monkeypatch.setattr(bench, "PROFILE_CEILINGS", out)
    assert bench.summarize_ceilings(tmp_path) == out
    text = out.read_text()
    for i, cap in enumerate(caps):
        assert f"| ceil_compress_mix_kernel | compress mix | {cap or '-'} | 4 | {10.0 * (i + 1):.2f} |" in text
    assert "| ceil_dequant_burst_kernel | dequantize-sum mix, workgroup bursts | - | 1 | 7.00 |" in text
    # launches that do not split evenly over the caps are an error, not a guess
    rows.append(("ceil_compress_mix_kernel", t, t + 5_000, 6240))
    _write_trace(tmp_path / "prof_ceilings" / "ceil_kernel_trace.csv", rows)
    with pytest.raises(ValueError):
        bench.summarize_ceilings(tmp_path)


def test_counter_rows_keep_the_instantiation_with_the_least_own_lds(tmp_path):
    """A counter CSV's dispatches of one kernel name but different template
    instantiations (told apart by the LDS the kernel declares) are not
    averaged together: the W = 8 dequantize-sum keeps its own rows."""
    sys.path.insert(0, str(ROOT))
    import bench
    import csv
    p = tmp_path / "c.csv"
    with open(p, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "LDS_Block_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for lds, v in ((21504, 10.0), (29696, 80.0), (21504, 12.0), (29696, 40.0)):
            w.writerow({"Kernel_Name": "decompress_ternary_vec_kernel", "LDS_Block_Size": lds,
                        "Counter_Name": "FETCH_SIZE", "Counter_Value": v})
        w.writerow({"Kernel_Name": "compress_ternary_vec_kernel", "LDS_Block_Size": 5120,
                    "Counter_Name": "FETCH_SIZE", "Counter_Value": 3.0})
    got = bench._read_counters_fewest_lds(p)
    assert got == {"decompress_ternary_vec_kernel": [10.0, 12.0],
                   "compress_ternary_vec_kernel": [3.0]}
    by_name = bench._read_counters_by_name(p)
    assert by_name["decompress_ternary_vec_kernel"]["FETCH_SIZE"] == [10.0, 12.0]
