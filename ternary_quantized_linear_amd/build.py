"""Builds libbitlinear.so (all HIP sources under csrc/) for gfx950 with hipcc.

Flags: -ffp-contract=off keeps every floating-point product and sum of the quantizers
as written (no FMA contraction), and fp32 division/sqrt stay correctly rounded; the
packed-fp32 feature is disabled so that no v_pk_*_f32 instructions are emitted. The
atomic optimizer is off: every atomic here is issued by one lane on purpose (row
combines, arrival counts), and the optimizer wrapped each in a scan over the active
lanes (the decode GEMV 3-7% faster without it).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbitlinear.so")
BUILD = os.path.join(HERE, "_build")
ARCH = os.environ.get("BITLINEAR_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-source additions: the decode GEMV and the skinny product take their leading scalar
# arguments (8 dwords) preloaded into SGPRs at wave launch.
PRELOAD8 = ["-mllvm", "-amdgpu-kernarg-preload-count=8"]
EXTRA = {"bl_gemv.hip": PRELOAD8, "bl_skinny.hip": PRELOAD8}


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA.get(os.path.basename(src), []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
