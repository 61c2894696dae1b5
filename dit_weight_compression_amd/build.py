"""Build the gfx950 HIP library in-tree with hipcc.

Produces dit_weight_compression_amd/libentropack_mi355x.so from csrc/*.hip.
Always recompiles (the caller decides when to build).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_NAME = "libentropack_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = [os.path.join(HERE, "csrc", "ep_decode.hip"), os.path.join(HERE, "csrc", "ep_encode_gpu.hip")]
ENC_LIB_PATH = os.path.join(HERE, "libentropack_encode.so")
ENC_SOURCES = [os.path.join(HERE, "csrc", "ep_encode.cpp")]
ENC_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra", "-I", os.path.join(ROOT, "include")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",           # y = x * g must round once, never fuse
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile the HIP decode library and the host encoder library."""
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC] + FLAGS + list(extra_flags or []) + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB_PATH)
    etmp = ENC_LIB_PATH + ".tmp"
    ecmd = ["g++"] + ENC_FLAGS + ENC_SOURCES + ["-o", etmp]
    if verbose:
        print(" ".join(ecmd), flush=True)
    subprocess.check_call(ecmd)
    os.replace(etmp, ENC_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
