"""The LDS reservation that caps resident workgroups per CU
(gradient_compression_quantize_amd/csrc/occupancy.h), checked on the host:
tests/occupancy_check.cpp is compiled with g++ and run. The GPU side of the
same fact (27,136 bytes per workgroup left room for 5 on a 160 KB CU, not 6;
sizes on the 2560-byte grid gave exactly 7, 6, 5, 4, 3 and 2) was measured
with workgroups that each wait a fixed time."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_reservation_allows_exactly_the_requested_workgroups(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    exe = tmp_path / "occupancy_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror",
                    "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    f"-I{ROOT / 'gradient_compression_quantize_amd' / 'csrc'}",
                    str(ROOT / "tests" / "occupancy_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip().endswith("OK"), res.stdout
