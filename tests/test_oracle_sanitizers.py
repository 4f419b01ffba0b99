"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
standalone C driver (tests/oracle_sanitize.c) compiled with oracle.c calls
every oracle function over edge-case sizes. A clean exit and no sanitizer
report are required. Memory safety and undefined behaviour only; the values
are pinned by the other oracle tests."""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_sanitize"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{ROOT / 'oracle'}", str(ROOT / "tests" / "oracle_sanitize.c"),
           str(ROOT / "oracle" / "oracle.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                       env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                            "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert r.returncode == 0, (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
    assert "sanitized oracle run: ok" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
