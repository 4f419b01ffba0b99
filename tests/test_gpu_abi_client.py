"""libgcq.so from a program that uses nothing but the C ABI and the HIP
runtime (tests/abi_client.cpp: its own hipMalloc'd buffers and stream, no
Python binding, no torch): the 2-bit error-feedback step, the QSGD-MN step
and the one-call GlobalRandK-MN step, every output bit-exact against the
oracle, plus one refused call."""
import subprocess

import pytest

from conftest import announce

pytestmark = pytest.mark.gpu


def test_c_abi_client_matches_the_oracle():
    import abi_client_build as acb
    if not acb.BIN.exists():
        pytest.fail(f"{acb.BIN} is not built: run python tests/abi_client_build.py (or build())")
    announce("C-ABI client (no Python binding, no torch)")
    res = subprocess.run([str(acb.BIN)], capture_output=True, text=True, timeout=110)
    print(res.stdout[-3000:], res.stderr[-2000:])
    assert res.returncode == 0 and res.stdout.strip().endswith("OK")
