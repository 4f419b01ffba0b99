"""Build libgcq.so (HIP, gfx950) in-tree with clang's HIP driver.

Each source compiles in two passes, so that device-only options stay off the
host compile:
  1. the device pass (gfx950 code object, bundled into a fat binary), with
     packed-fp32 VALU instructions disabled;
  2. the host pass, which embeds that fat binary and registers its kernels.
Both passes get the same compilation-unit id (-cuid), so that names of
file-scope device variables agree between the code object and the host
registration. The objects are then linked into one shared library.
"""
from __future__ import annotations

import hashlib
import os
import pathlib
import subprocess

PKG = pathlib.Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIB_PATH = PKG / "libgcq.so"
CEILINGS_LIB_PATH = PKG / "libgcq_ceilings.so"
BUILD_DIR = PKG / "_build"

SOURCES = ["status.hip", "twobit.hip", "ternary.hip", "qsgd.hip"]
# the benchmark's HBM ceiling kernels: a library of their own
CEILINGS_SOURCES = ["hbm_ceilings.hip"]

# Options of both passes.
COMMON_FLAGS = [
    "-x", "hip",
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    # fp32 is evaluated one operation at a time: no contraction into FMA
    "-ffp-contract=off",
    "-Wall",
]

# Device pass only: no packed-fp32 VALU instructions (v_pk_add/mul/fma_f32).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def clang() -> str:
    return os.path.join(rocm(), "lib", "llvm", "bin", "clang++")


def hipcc() -> str:
    return os.path.join(rocm(), "bin", "hipcc")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(str(c) for c in cmd), flush=True)
    subprocess.run([str(c) for c in cmd], check=True)


def compile_source(src: pathlib.Path, out_dir: pathlib.Path, includes, verbose: bool = False,
                   extra=()) -> pathlib.Path:
    """Device pass, then host pass with the fat binary embedded; returns the
    host object."""
    cuid = hashlib.sha256(src.name.encode()).hexdigest()[:16]
    fatbin = out_dir / (src.stem + ".hipfb")
    obj = out_dir / (src.stem + ".o")
    inc = [f"-I{d}" for d in includes]
    _run([clang(), *COMMON_FLAGS, *extra, *DEVICE_FLAGS, f"-cuid={cuid}", *inc,
          "--offload-device-only", "-c", src, "-o", fatbin], verbose)
    _run([clang(), *COMMON_FLAGS, *extra, f"-cuid={cuid}", *inc, "--offload-host-only",
          "-Xclang", "-fcuda-include-gpubinary", "-Xclang", fatbin, "-c", src, "-o", obj],
         verbose)
    return obj


def link_shared(objs, lib_path: pathlib.Path, verbose: bool = False) -> pathlib.Path:
    tmp = lib_path.with_suffix(".so.tmp%d" % os.getpid())
    _run([hipcc(), "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, lib_path)
    return lib_path


def build(verbose: bool = False) -> pathlib.Path:
    """Compile every HIP source into libgcq.so, and the benchmark's ceiling
    kernels into libgcq_ceilings.so (always recompiles)."""
    out = BUILD_DIR / "gcq"
    out.mkdir(parents=True, exist_ok=True)
    objs = [compile_source(CSRC / s, out, (INCLUDE, CSRC), verbose) for s in SOURCES]
    link_shared(objs, LIB_PATH, verbose)
    cout = BUILD_DIR / "ceilings"
    cout.mkdir(parents=True, exist_ok=True)
    cobjs = [compile_source(CSRC / s, cout, (INCLUDE,), verbose) for s in CEILINGS_SOURCES]
    link_shared(cobjs, CEILINGS_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
