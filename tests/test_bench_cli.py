"""bench.py's command-line contract, on the CPU: more than one GPU is
refused with a message (this library runs on one GPU), and a run with no
GPU visible fails with a message instead of printing a result line. Also
the rule that names a kernel's roofline bound."""
import json
import os
import pathlib
import subprocess
import sys

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
