"""Pins for the oracle's Philox4x32-10 (Salmon et al., SC'11).

The oracle's bijection is compared with two independent open-source
implementations installed in this image -- PyTorch's header-only
at::philox_engine and rocRAND's philox4x32_10_engine -- each compiled into a
small host-only helper (tests/xcheck/*.cpp). Neither helper is linked into the
oracle or the HIP library. A chi-square check covers output uniformity.
"""
import pathlib
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle

XCHECK = pathlib.Path(__file__).resolve().parent / "xcheck"
TORCH_INC = None
try:
    import torch  # noqa: F401
    TORCH_INC = pathlib.Path(torch.__file__).resolve().parent / "include"
except Exception:
    pass


def _compile(tmp_path_factory, src: str, cmd_prefix) -> pathlib.Path:
    out = tmp_path_factory.mktemp("xcheck") / pathlib.Path(src).stem
    subprocess.run([*cmd_prefix, str(XCHECK / src), "-o", str(out)], check=True,
                   capture_output=True)
    return out


def _run(exe: pathlib.Path, lines) -> np.ndarray:
    res = subprocess.run([str(exe)], input="\n".join(lines) + "\n", text=True,
                         capture_output=True, check=True)
    return np.array([[int(v) for v in ln.split()] for ln in res.stdout.strip().splitlines()],
                    dtype=np.uint64)


def _random_cases(m: int, seed: int):
    rng = np.random.default_rng(seed)
    ctr = rng.integers(0, 2 ** 32, size=(m, 4), dtype=np.uint64)
    key = rng.integers(0, 2 ** 32, size=(m, 2), dtype=np.uint64)
    # a few structured corners
    ctr[0] = 0
    key[0] = 0
    ctr[1] = 2 ** 32 - 1
    key[1] = 2 ** 32 - 1
    ctr[2] = [4, 0, 7, 0]
    key[2] = [12345, 0]
    return ctr, key


def _oracle_block(ctr, key) -> np.ndarray:
    return np.array([oracle.philox4x32_10(c, k) for c, k in zip(ctr, key)], dtype=np.uint64)


@pytest.mark.skipif(TORCH_INC is None or shutil.which("g++") is None,
                    reason="torch headers or g++ unavailable")
def test_philox_matches_pytorch_engine(tmp_path_factory):
    exe = _compile(tmp_path_factory, "philox_torch.cpp",
                   ["g++", "-std=c++17", "-O1", f"-I{TORCH_INC}"])
    ctr, key = _random_cases(3000, 1)
    # torch's engine: key = seed; counter = (offset, subsequence) as 2x64 bit
    seeds = (key[:, 1] << np.uint64(32)) | key[:, 0]
    offs = (ctr[:, 1] << np.uint64(32)) | ctr[:, 0]
    subs = (ctr[:, 3] << np.uint64(32)) | ctr[:, 2]
    got = _run(exe, [f"{int(s)} {int(b)} {int(o)}" for s, b, o in zip(seeds, subs, offs)])
    np.testing.assert_array_equal(_oracle_block(ctr, key), got)


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc unavailable")
def test_philox_matches_rocrand_engine(tmp_path_factory):
    exe = _compile(tmp_path_factory, "philox_rocrand.cpp",
                   ["hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1"])
    ctr, key = _random_cases(3000, 2)
    got = _run(exe, [" ".join(str(int(v)) for v in (*c, *k)) for c, k in zip(ctr, key)])
    np.testing.assert_array_equal(_oracle_block(ctr, key), got)


def test_philox_output_is_uniform():
    """Top byte of 4 x 20000 outputs over consecutive counters: chi-square
    over 256 bins, far from any rejection threshold."""
    words = np.concatenate([oracle.philox4x32_10([i, 0, 3, 0], [77, 0]) for i in range(20000)])
    hist = np.bincount((words >> 24).astype(np.int64), minlength=256)
    chi2 = stats.chisquare(hist).statistic
    assert chi2 < stats.chi2.ppf(1 - 1e-6, 255)


def test_philox_is_a_function_of_every_input_word():
    base_c, base_k = [1, 2, 3, 4], [5, 6]
    ref = oracle.philox4x32_10(base_c, base_k)
    for i in range(4):
        c = list(base_c)
        c[i] ^= 1
        assert not np.array_equal(oracle.philox4x32_10(c, base_k), ref)
    for i in range(2):
        k = list(base_k)
        k[i] ^= 1
        assert not np.array_equal(oracle.philox4x32_10(base_c, k), ref)
