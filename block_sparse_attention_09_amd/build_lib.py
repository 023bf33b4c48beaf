"""Builds libabatt.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libabatt.so")

SOURCES = ["key_means.hip", "kmeans.hip", "score.hip", "sampler.hip", "sampler_onepass.hip", "attend.hip", "scratch.hip",
           "abatt.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # no packed fp32 (v_pk_*_f32) instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# per-file flags: the attention kernels never see NaN by construction, and
# without NaN semantics fmax needs no canonicalising moves around MFMA results
FILE_FLAGS = {"attend.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


PROBE_SRC = os.path.join(CSRC, "mfma_probe.hip")
PROBE = os.path.join(PKG, "mfma_probe")


def build_probe() -> str:
    """The MFMA issue probe (a measurement program, not part of libabatt)."""
    cmd = [HIPCC, *FLAGS, PROBE_SRC, "-o", PROBE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for mfma_probe.hip:\n{r.stderr}")
    return PROBE


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    if verbose:
        print(f"built {LIB} and {PROBE}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
