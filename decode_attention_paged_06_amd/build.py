"""Build libpagedattn.so in-tree with hipcc for gfx950.

    python -m decode_attention_paged_06_amd.build

Every call recompiles all sources (objects go to _build/ next to this file).
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libpagedattn.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)

SOURCES = [
    "host/api.cpp",
    "kernels/decode_valu.hip",
    "kernels/decode_mfma.hip",
    "kernels/reduce.hip",
    "kernels/gather.hip",
]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed-fp32 VALU forms are disabled for all device code.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, src.replace("/", "_") + ".o")
    cmd = [_hipcc()] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()
