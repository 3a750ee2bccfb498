"""Build libqsa.so (the C ABI plus the HIP kernels) for gfx950, in tree.

    python -m block_sparse_attention_c4_amd.build [--debug]

--debug builds libqsa_debug.so instead: the same library compiled with -DQSA_DEBUG,
whose kernels trap when device-side contents (page-table entries, positions,
counts) break their documented ranges.  Point QSA_LIB at it to use it.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqsa.so")
OUT_DEBUG = os.path.join(PKG, "libqsa_debug.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["qsa_api.cpp", "qsa_build.hip", "qsa_index.hip", "qsa_topk.hip", "qsa_prefill.hip",
           "qsa_attn.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # packed FP32 forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(src: str, debug: bool = False) -> str:
    obj = os.path.join(OBJ, "debug" if debug else "", os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DQSA_DEBUG"] if debug else []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, debug: bool = False) -> str:
    out = OUT_DEBUG if debug else OUT
    os.makedirs(os.path.join(OBJ, "debug" if debug else ""), exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, debug), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
