"""Build libmiattn.so in-tree with hipcc for gfx950.

    python -m online_softmax_monoid_amd.build

Every HIP source is compiled for gfx950 only, with packed-FP32 instruction
selection turned off (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmiattn.so")
SOURCES = ["api.cpp", "prefill.hip", "prefill_q64.hip", "prefill_pingpong.hip", "decode.hip",
           "backward.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the online-softmax rescale and the
            # epilogue touch them with VALU ops, which cannot address AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *extra]


def build(out: str = LIB, extra=(), verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        p = os.path.join(CSRC, s)
        srcs += ["-x", "hip", p]
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *flags(extra), "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if msg.strip() and verbose:
        print(msg)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
