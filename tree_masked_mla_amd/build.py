"""Build libddtv.so (HIP, gfx950 only) in-tree with hipcc.

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

SOURCES = ["api.hip", "visibility.hip", "attn_valu.hip", "attn_mfma.hip", "attn_mfma_bf16.hip", "merge.hip",
           "tree_build.hip", "tree_accept.hip", "tail.hip", "neighbour.hip"]
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


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link the shared library.  Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
