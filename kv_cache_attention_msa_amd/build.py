"""Build libmsa.so (the C-ABI library) from csrc/*.hip with hipcc for gfx950.

Each translation unit is compiled to an object in parallel, then linked into
kv_cache_attention_msa_amd/libmsa.so, next to the Python binding.  The same
build also links libmsa_peaks.so from peaks/*.hip: a measuring instrument
for the bench (the matrix-core rate of the GPU), not part of the attention
path.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmsa.so")
PEAKS = os.path.join(HERE, "peaks")
PEAKS_LIB = os.path.join(HERE, "libmsa_peaks.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-FP32 VALU forms
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs (gfx950 allows it): the online softmax
    # rescales them with plain VALU ops instead of AGPR round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build_peaks() -> str:
    """Compile peaks/*.hip and link libmsa_peaks.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(PEAKS, f) for f in os.listdir(PEAKS) if f.endswith(".hip"))
    objs = []
    for src in srcs:
        obj = os.path.join(BUILD, "peaks_" + os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        objs.append(obj)
    _link(objs, PEAKS_LIB)
    return PEAKS_LIB


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every csrc/*.hip and link libmsa.so, then libmsa_peaks.so;
    returns the path of libmsa.so."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), srcs))
    objs = [o for o, _ in results]
    if verbose:
        for _, err in results:
            if err.strip():
                print(err, file=sys.stderr)
    _link(objs, LIB)
    build_peaks()
    return LIB


def clean():
    shutil.rmtree(BUILD, ignore_errors=True)
    for f in (LIB, PEAKS_LIB):
        if os.path.exists(f):
            os.remove(f)


if __name__ == "__main__":
    print(build(verbose=True))
