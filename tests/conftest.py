import os
import pathlib
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

GOLDEN = ROOT / "tests" / "golden"


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: full-size parity case (seconds to a minute)")


@pytest.fixture(scope="session")
def golden_dir():
    return GOLDEN


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def gcq():
    """The HIP library's Python binding. GPU tests fail (not skip) when the
    library is missing: a GPU run must exercise the native path."""
    if not gpu_available():
        pytest.skip("no GPU visible")
    import gradient_compression_quantize_amd as gcq_mod
    gcq_mod.load()  # raises if libgcq.so is missing
    return gcq_mod


def announce(msg: str) -> None:
    """Flush a line naming the case before a GPU step runs."""
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()
    sys.stderr.write(f"[case] {msg}\n")
    sys.stderr.flush()
