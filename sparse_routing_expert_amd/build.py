"""Build libmoe.so (HIP kernels + C ABI) in-tree for gfx950 with hipcc.

    python -m sparse_routing_expert_amd.build

Compiles every source under csrc/ to an object in parallel, links them into
sparse_routing_expert_amd/libmoe.so, and replaces the library atomically.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libmoe.so")
SOURCES = ["route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "backward.hip", "noalloc.hip", "probes.hip", "moe_api.cpp"]
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
    # keep the compiler from forming packed fp32 arithmetic (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *COMMON_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        objs = [os.path.join(tmp, s + ".o") for s in SOURCES]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
            list(ex.map(_compile, SOURCES, objs))
        out_tmp = os.path.join(tmp, "libmoe.so")
        cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        shutil.copyfile(out_tmp, LIB_PATH + ".tmp")
        os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
