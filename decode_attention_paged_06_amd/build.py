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
    "kernels/prefill_mfma32.hip",
    "kernels/reduce.hip",
    "kernels/gather.hip",
    "kernels/schedule.hip",
    "kernels/scratch.hip",
    "kernels/probe.hip",
]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}"]
# Packed-fp32 VALU forms are disabled for all device code.  MFMA results stay
# in ordinary VGPRs: the decode loop rescales its P.V accumulators with VALU
# multiplies every tile, and accumulators kept in AGPRs would need a copy to
# VGPRs and back around each rescale.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found")
    return path


def _compile(src: str, csrc: str = CSRC, build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, src.replace("/", "_") + ".o")
    cmd = [_hipcc()] + COMMON + [f"-I{csrc}"]
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    cmd += ["-c", os.path.join(csrc, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = True, csrc: str = CSRC, out: str = LIB_PATH) -> str:
    """Compile `csrc` (default: this package's sources) into the shared library `out`."""
    build_dir = BUILD_DIR if csrc == CSRC else os.path.join(os.path.dirname(out), "_build")
    os.makedirs(build_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, csrc, build_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    import argparse

    ap = argparse.ArgumentParser()
    ap.add_argument("--csrc", default=CSRC, help="source tree (default: this package's csrc/)")
    ap.add_argument("--out", default=LIB_PATH, help="output shared library")
    ns = ap.parse_args()
    build(csrc=os.path.abspath(ns.csrc), out=os.path.abspath(ns.out))
