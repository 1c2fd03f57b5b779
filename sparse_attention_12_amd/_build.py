"""Build the gfx950 HIP library libdsa_mla.so in-tree with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdsa_mla.so")
DEBUG_LIB = os.path.join(HERE, "libdsa_mla_debug.so")  # the same sources with -DDSA_DEBUG
SOURCES = ["abi.hip", "noalloc.hip", "plan.cpp", "indexer.hip", "topk.hip", "mla.hip", "rope.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _compile(job) -> str:
    src, debug = job
    obj = os.path.join(BUILD, src + (".debug.o" if debug else ".o"))
    cmd = [HIPCC, *FLAGS, *(["-DDSA_DEBUG"] if debug else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}{' (debug)' if debug else ''}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile every HIP source for gfx950 and link libdsa_mla.so, and with
    debug also libdsa_mla_debug.so (the kernels' checks compiled in); always
    rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = [(s, False) for s in SOURCES] + ([(s, True) for s in SOURCES] if debug else [])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 8)) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    if verbose:
        print(f"built {LIB}")
    if debug:
        _link(objs[len(SOURCES):], DEBUG_LIB)
        if verbose:
            print(f"built {DEBUG_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
