"""Builds libidattn.so in-tree with hipcc for gfx950.

    python -m fixed_state_ssm_amd.build [--verbose]

Each source is compiled to an object of its own (in parallel), then the
objects are linked into one shared library.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libidattn.so")
OBJ_DIR = os.path.join(PKG, "_build")
SOURCES = ["api.cpp", "featmap.hip", "scan_seq.hip", "chunked_ws.hip", "decode.hip", "backward.hip", "noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    return res.returncode, out


def build(verbose: bool = False) -> str:
    """Compile every HIP/C++ source into one shared library; returns its path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".o") for s in srcs]
    jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)), 16)
    with concurrent.futures.ThreadPoolExecutor(max(jobs, 1)) as ex:
        results = list(ex.map(lambda so: _run([HIPCC, *FLAGS, "-c", so[0], "-o", so[1]], verbose),
                              zip(srcs, objs)))
    for (rc, out), src in zip(results, srcs):
        if rc != 0:
            raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({rc}):\n{out}")
        if verbose and out.strip():
            print(out, flush=True)
    tmp = LIB + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
