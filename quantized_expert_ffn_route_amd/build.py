"""Build the HIP library ``libmoe.so`` in-tree for gfx950 (MI355X).

    python -m quantized_expert_ffn_route_amd.build

Compiles every source under ``csrc/`` with hipcc and links the shared
library next to this file.  Device code is built with packed-fp32 ops
disabled and with hardware float atomics; the host packer is built without
FP contraction so each step of the block quantiser is one IEEE rounding.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")

ARCH = "gfx950"
DEVICE_SOURCES = ["kernels_route.hip", "kernels_decode.hip", "kernels_prefill.hip",
                  "kernels_dense.hip", "scratch.hip"]
HOST_SOURCES = ["moe_abi.cpp", "pack.cpp"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _common():
    return ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if src.endswith(".hip"):
        cmd = [_hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-munsafe-fp-atomics",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               *_common(), "-c", path, "-o", obj]
    else:
        # host-only translation unit (no device code)
        cmd = [_hipcc(), "-x", "c++", "-ffp-contract=off", "-D__HIP_PLATFORM_AMD__",
               f"-I{os.path.join(_rocm(), 'include')}",
               *_common(), "-c", path, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link ``libmoe.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = DEVICE_SOURCES + HOST_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs, "-lpthread"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
