"""Builds the HIP library libtre_moe.so in-tree with hipcc for gfx950.

Run as `python -m token_routed_expert_amd.build` (or via __graft_entry__.build()).
Every call recompiles all sources: objects go to token_routed_expert_amd/_build/,
the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtre_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    # no packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]

_BENIGN = "'-packed-fp32-ops' is not a recognized feature for this target"

# Per-file additions.  probe.hip: MFMAs accumulate in VGPRs (with the default
# accumulator-register form the compiler moves the accumulators between
# register files on every loop trip, and the probe would time those moves).
EXTRA_FLAGS = {"probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if _BENIGN not in l and "(ignoring feature)" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        outs = list(ex.map(lambda so: _run([HIPCC, *CXXFLAGS,
                                            *EXTRA_FLAGS.get(os.path.basename(so[0]), []),
                                            "-c", so[0], "-o", so[1]]),
                           zip(srcs, objs)))
    if verbose:
        for o in outs:
            if o:
                print(o, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
