"""Build libgcq.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import pathlib
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_PATH = PKG / "libgcq.so"

SOURCES = ["status.hip", "twobit.hip", "ternary.hip", "qsgd.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # fp32 is evaluated one operation at a time: no contraction into FMA
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every HIP source into libgcq.so (always recompiles)."""
    tmp = LIB_PATH.with_suffix(".so.tmp%d" % os.getpid())
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *[str(CSRC / s) for s in SOURCES], "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
