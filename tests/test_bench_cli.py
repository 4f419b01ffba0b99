"""bench.py's command-line contract, on the CPU: more than one GPU is
refused with a message (this library runs on one GPU), and a run with no
GPU visible fails with a message instead of printing a result line."""
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
