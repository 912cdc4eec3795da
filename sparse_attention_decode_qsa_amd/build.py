"""Build libqsa.so (HIP kernels + C ABI) and libqsa_calib.so (the counter-calibration copy)
for gfx950 with hipcc, in-tree.

    python -m sparse_attention_decode_qsa_amd.build
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqsa.so")
SOURCES = ["index_score.hip", "index_score_mq.hip", "topk_select.hip", "sparse_attn.hip", "lse_merge.hip", "check_pages.hip",
           "side_cache.hip", "qsa_api.hip"]
CALIB_LIB = os.path.join(PKG, "libqsa_calib.so")
CALIB_SOURCES = ["calib_copy.hip"]
ARCH = "gfx950"

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every kernel source and link libqsa.so and libqsa_calib.so; returns libqsa's path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + len(CALIB_SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES + CALIB_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
