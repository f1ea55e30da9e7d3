"""Build ``libnvfp4ffn.so`` (the C-ABI library) for gfx950 with hipcc.

``python -m nvfp4_weight_dense_amd.build`` compiles every ``csrc/*.hip``
to an object in ``_build/`` and links them into the package directory.
Cross-compiles without a GPU.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB_NAME = "libnvfp4ffn.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
    f"-I{CSRC}",
    # no packed-FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE fp32 division/sqrt and denormals: the quantizer is bit-exact
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and noise not in ln]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    """Compile and link the library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    # A kernel template whose host-side instantiation failed leaves its launch
    # stub undefined without any compile error; binding every symbol now (in
    # a child process, so this one keeps no handle) turns that into a build
    # failure instead of a load failure later.
    chk = subprocess.run(
        [sys.executable, "-c", "import ctypes, os, sys; ctypes.CDLL(sys.argv[1], os.RTLD_NOW)", tmp],
        capture_output=True, text=True)
    if chk.returncode != 0:
        raise RuntimeError(f"built library does not load:\n{chk.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def clean() -> None:
    shutil.rmtree(BUILD, ignore_errors=True)


if __name__ == "__main__":
    build(verbose=True)
