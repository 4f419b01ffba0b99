"""Builds tests/_bin/abi_client from tests/abi_client.cpp: a host-only C++
program that calls libgcq.so through include/gcq.h and checks it against
the oracle (oracle/liboracle.so). Both libraries must be built first; the
binary finds them through a RUNPATH relative to itself, so the tree can move.
"""
from __future__ import annotations

import os
import pathlib
import subprocess

ROOT = pathlib.Path(__file__).resolve().parent.parent
SRC = ROOT / "tests" / "abi_client.cpp"
BIN = ROOT / "tests" / "_bin" / "abi_client"


def build(verbose: bool = False) -> pathlib.Path:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    BIN.parent.mkdir(parents=True, exist_ok=True)
    tmp = BIN.with_name(BIN.name + f".tmp{os.getpid()}")
    cmd = ["g++", "-std=c++17", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{rocm}/include", f"-I{ROOT / 'include'}", f"-I{ROOT / 'oracle'}", str(SRC),
           "-o", str(tmp),
           f"-L{ROOT / 'gradient_compression_quantize_amd'}", "-lgcq",
           f"-L{ROOT / 'oracle'}", "-loracle", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gradient_compression_quantize_amd:$ORIGIN/../../oracle:"
           f"{rocm}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
