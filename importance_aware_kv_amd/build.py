"""Build the HIP library libhikv.so in-tree for gfx950.

    python -m importance_aware_kv_amd.build

hipcc cross-compiles the device code, so this also works on a machine with no
GPU.  Packed-FP32 instruction selection is switched off for every kernel.
"""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libhikv.so")
SOURCES = ["api.hip", "decode.hip", "step.hip", "stage2.hip", "prefill.hip"]
# measurement aids for the benchmark (a streaming read, an empty kernel): a
# library of their own, not part of the decode path
CALIB_LIB = os.path.join(PKG, "libhikv_calib.so")
CALIB_SOURCES = ["calib.hip"]
ARCH = os.environ.get("HIKV_ARCH", "gfx950")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results and accumulators in ordinary VGPRs: the attention
    # kernel's outputs are also rescaled by vector instructions, and with
    # accumulation registers the compiler copies them back and forth around
    # every P.V step.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + CFLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print(LIB)
        print(CALIB_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
