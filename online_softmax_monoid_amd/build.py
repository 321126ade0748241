"""Build libmiattn.so (the attention library) and libmiprobe.so (the machine
probes the benchmark reports beside it) in-tree with hipcc for gfx950.

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
SOURCES = ["api.cpp", "prefill_d64.hip", "prefill_d128.hip", "prefill_d256.hip", "decode.hip",
           "backward.hip"]
PROBE_LIB = os.path.join(PKG, "libmiprobe.so")
PROBE_SOURCES = ["probes.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in VGPRs: the online-softmax rescale and the
            # epilogue touch them with VALU ops, which cannot address AGPRs
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, *extra]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln)
    return res.returncode, msg


def build(out: str = LIB, extra=(), verbose: bool = False, probes: bool = True) -> str:
    """Build the attention library at `out` and, unless probes is False, the
    probe library beside the package; returns `out`."""
    _build_lib(out, SOURCES, extra, verbose)
    if probes:
        _build_lib(PROBE_LIB, PROBE_SOURCES, extra, verbose)
    return out


def _build_lib(out, sources, extra=(), verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the shared
    library; the objects live in a build folder next to the sources."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    tag = "%d" % os.getpid()
    cmds, objs = [], []
    for s in sources:
        obj = os.path.join(objdir, os.path.splitext(s)[0] + "." + tag + ".o")
        objs.append(obj)
        cmds.append([hipcc(), *flags(extra), "-c", "-o", obj, "-x", "hip", os.path.join(CSRC, s)])
    workers = max(1, min(len(cmds), os.cpu_count() or 1, 8))
    try:
        with ThreadPoolExecutor(workers) as pool:
            results = list(pool.map(_run, cmds))
        for cmd, (rc, msg) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + msg)
            if msg.strip() and verbose:
                print(msg)
        tmp = out + ".tmp" + tag
        rc, msg = _run([hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
        if rc != 0:
            raise RuntimeError("link failed:\n" + msg)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
