"""Build libconvrot.so in-tree with hipcc for gfx950.

Usage: python -m hadamard_rotated_int8_amd.build  (or build() from Python)

Every call recompiles all sources: objects go to _build/ at the repository
root, the shared libraries next to this file.  Besides the layer's library,
libconvrot_ceiling.so holds the measurement kernel the benchmark times
beside the GEMM (include/convrot_ceiling.h); nothing on the hot path uses it.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libconvrot.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
CEILING_LIB_PATH = os.path.join(PKG_DIR, "libconvrot_ceiling.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "pack.hip", "wprep.hip", "gemm.hip", "gemm_small.hip", "lora.hip"]
CEILING_SOURCES = ["ceiling.hip"]

# Packed-FP32 instructions are kept out of generated code on purpose.
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
    cmd = [_hipcc(), *COMMON_FLAGS, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # surface warnings other than the host pass's note about the GPU-only feature
    noise = ("packed-fp32-ops", "warning generated", "warnings generated")
    msgs = [ln for ln in r.stderr.splitlines() if ln.strip() and not any(n in ln for n in noise)]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(extra_flags: list[str] | None = None, verbose: bool = False) -> str:
    """Compile every source, link libconvrot.so and libconvrot_ceiling.so;
    returns the path of libconvrot.so."""
    extra = list(extra_flags or [])
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = SOURCES + CEILING_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(sources), 8)) as ex:
        objs = dict(zip(sources, ex.map(lambda s: _compile(s, extra), sources)))
    _link([objs[s] for s in SOURCES], LIB_PATH)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {CEILING_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
