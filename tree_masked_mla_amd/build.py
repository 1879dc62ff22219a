"""Build libddtv.so (HIP, gfx950 only) in-tree with hipcc, and libddtv_calib.so,
the benchmark's HBM read-stream calibration (not part of the verify path).

    python -m tree_masked_mla_amd.build

Every HIP translation unit is compiled with packed-FP32 instruction selection
disabled (the compiler still emits scalar FP32 FMAs); kernels target gfx950
(MI355X, CDNA4) and nothing else.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libddtv.so")
CALIB_LIB = os.path.join(PKG, "libddtv_calib.so")

SOURCES = ["api.hip", "visibility.hip", "attn_valu.hip", "attn_mfma.hip", "attn_mfma_bf16.hip", "merge.hip",
           "tree_build.hip", "tree_accept.hip", "tail.hip", "neighbour.hip"]
CALIB_SOURCES = ["calib_stream.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature and says so; keep other warnings.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    rest = "\n".join(l for l in r.stderr.splitlines() if noise not in l).strip()
    if rest:
        sys.stderr.write(rest + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link both shared libraries.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
