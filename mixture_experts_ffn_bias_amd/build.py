"""Compile the gfx950 HIP sources into libmoe.so, next to this file.

    python -m mixture_experts_ffn_bias_amd.build

Every call recompiles (one hipcc process per source file, in parallel) and
links.  Flags: gfx950 only, -O3, and packed fp32 instructions disabled
(``-packed-fp32-ops``) so that the compiler never forms v_pk_* fp32 ops.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["api.hip", "gate.hip", "permute.hip", "ffn.hip", "combine.hip", "norm.hip", "decode.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is expected
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, jobs: int = 8) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs, cmds = [], []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([cc, *FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(jobs, len(cmds))) as ex:
        for cmd, out in zip(cmds, ex.map(_run, cmds)):
            if verbose and out:
                print(out, file=sys.stderr)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
