"""Build the device probes beside the tests: tests/probes/_build/libgla_probes.so.

The probes check, on the device, assumptions that the library's kernels are
built on (the LDS transpose-read lane layout) and measure the practical HBM
ceilings quoted with the roofline.  They are never linked into libgla.so.
Usage: ``python tests/probes/build.py`` (also run by ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "_build", "libgla_probes.so")


def build(verbose: bool = False) -> str:
    sys.path.insert(0, ROOT)
    from recurrent_vision_backbone_key_amd import build as libbuild
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [libbuild.HIPCC] + libbuild.HIP_FLAGS + ["-shared", os.path.join(HERE, "gla_probes.hip"), "-o", tmp]
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError("probe build failed: " + " ".join(cmd))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
