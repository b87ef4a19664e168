"""Build the HIP library libra.so in-tree for gfx950 with hipcc, and its
debug build libra_debug.so (-DRA_DEBUG: bounds checks at the decode
kernels' computed global accesses, reported in the workspace, never a trap).

    python top_sparse_attention_gqa_amd/build.py

Run as a script (not with -m): the package itself loads the library.

Always recompiles. Objects go to ``_build/`` (git-ignored); the shared
libraries land next to this file, where the binding (and the debug-build
test) load them.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libra.so")
LIB_DEBUG = os.path.join(PKG, "libra_debug.so")

SOURCES = ["ra_api.cpp", "kv_append.hip", "score_scan.hip", "topk_select.hip",
           "gather_attn.hip", "prefill_topk.hip", "graph_search.hip", "sparse_attend.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are switched off for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function"]


def _compile(src: str, debug: bool = False) -> str:
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, "debug" if debug else "", src + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    extra = ["-DRA_DEBUG"] if debug else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, *lang, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile libra.so (and, with debug=True, libra_debug.so)."""
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if debug else [])
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    _link(objs[:len(SOURCES)], LIB)
    if debug:
        _link(objs[len(SOURCES):], LIB_DEBUG)
    if verbose:
        print(f"built {LIB}" + (f" and {LIB_DEBUG}" if debug else ""))
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
