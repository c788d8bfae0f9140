"""Build the HIP library in-tree: recurrent_vision_backbone_key_amd/_lib/libgla.so.

The host-side argument checks (gla_plan.cpp) are compiled with g++ without
any HIP header; the kernels and the C-ABI layer are compiled with hipcc for
gfx950 only.  Usage: ``python -m recurrent_vision_backbone_key_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libgla.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX_HOST", shutil.which("g++") or "g++")

HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
             # keep hipcc from forming packed-fp32 instructions
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I" + INCLUDE, "-I" + CSRC]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-I" + INCLUDE, "-I" + CSRC]

# (source, compiler) -- the generic kernels are instantiated in four units
# (storage type x square / mixed head sizes) that compile in parallel.
UNITS = [
    ("gla_plan.cpp", "host", []),
    ("gla_api.cpp", "hip", []),
    ("gla_kernel.hip", "hip", []),
    ("gla_chunk_f16.hip", "hip", []),
    ("gla_chunk_f32.hip", "hip", []),
    ("gla_chunk_f16_mixed.hip", "hip", []),
    ("gla_chunk_f32_mixed.hip", "hip", []),
    ("gla_onepass.hip", "hip", []),
    ("gla_wide.hip", "hip", []),
    ("gla_proj.hip", "hip", []),
    ("gla_proj_bwd.hip", "hip", []),
    ("gla_sswiglu.hip", "hip", []),
    ("gla_bwd.hip", "hip", []),
    ("gla_noalloc.hip", "hip", []),
]


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    # hipcc's host pass reports the packed-fp32 feature flag as unknown: harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l)
    if msg.strip():
        sys.stderr.write(msg + "\n")


def _compile(src, kind, extra):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    if kind == "host":
        cmd = [CXX] + HOST_FLAGS + extra + ["-c", path, "-o", obj]
    else:
        cmd = [HIPCC] + HIP_FLAGS + extra + ["-c", path, "-o", obj]
    _run(cmd)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(UNITS))) as ex:
        objs = list(ex.map(lambda u: _compile(*u), UNITS))
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
