"""Build libattn.so in-tree: hipcc, gfx950 only, ahead of time (no JIT).

    python -m tiled_attention_05_amd.build        # or __graft_entry__.build()

Every HIP source is compiled with packed-fp32 instruction selection disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the host-only C ABI
file is plain C++.  Objects go to ``_build/`` at the repository root and the
shared library lands next to this file, where ``_lib.load()`` finds it.

A second library, ``libattn_single_stage.so``, is linked from the same objects
except the two forward kernels, which are compiled with ``-DATTN_SINGLE_STAGE``:
one key/value tile in flight and every copy waited for as soon as it is
issued. It exists for the tests only, which require its results to equal the
pipelined library's bit for bit (a missing wait or a buffer reused too early
shows up as a difference).
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
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn.so")
LIB_SINGLE_STAGE = os.path.join(PKG, "libattn_single_stage.so")
SINGLE_STAGE_SOURCES = ("attn_fwd_bf16.hip", "fp8.hip")   # the sources that read ATTN_SINGLE_STAGE
ARCH = "gfx950"

HIP_FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src, hipcc, extra, tag=""):
    obj = os.path.join(OBJ, os.path.basename(src) + tag + ".o")
    if src.endswith(".hip"):
        cmd = [hipcc, *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    else:
        cmd = [hipcc, *CXX_FLAGS, "-D__HIP_PLATFORM_AMD__", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(hipcc, objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, extra=(), single_stage: bool = True) -> str:
    """Compile every source and link libattn.so (and, unless single_stage is
    False, libattn_single_stage.so); returns the path of libattn.so."""
    hipcc = _hipcc()
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = [(s, list(extra), "") for s in srcs]
    if single_stage:
        jobs += [(s, list(extra) + ["-DATTN_SINGLE_STAGE"], ".single_stage") for s in srcs
                 if os.path.basename(s) in SINGLE_STAGE_SOURCES]
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 4, 8)) as ex:
        objs = list(ex.map(lambda j: _compile(j[0], hipcc, j[1], j[2]), jobs))
    _link(hipcc, objs[:len(srcs)], LIB)
    if single_stage:
        alt = dict(zip((os.path.basename(s) for s, _, _ in jobs[len(srcs):]), objs[len(srcs):]))
        _link(hipcc, [alt.get(os.path.basename(s), o) for s, o in zip(srcs, objs[:len(srcs)])], LIB_SINGLE_STAGE)
    if verbose:
        print(f"built {LIB}" + (f" and {os.path.basename(LIB_SINGLE_STAGE)}" if single_stage else "")
              + f" from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
