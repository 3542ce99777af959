"""Ahead-of-time build of the gfx950 library ``libnvfp4.so`` with hipcc.

Run ``python -m grouped_gemm_nvfp4_amd.build`` (or ``__graft_entry__.build()``).
The library lands next to this file, so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4.so")

SOURCES = ["api.cpp", "kernels.hip", "kernels_dma.hip", "kernels_dma_one.hip", "kernels_dma_special.hip",
           "kernels_dma_four.hip", "kernels_wide.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _quiet(text: str) -> str:
    # hipcc's host pass does not know the packed-fp32 feature: harmless
    return "\n".join(l for l in text.splitlines() if "is not a recognized feature for this target" not in l)


def build(verbose: bool = False) -> str:
    """Compile every source into ``libnvfp4.so`` (always recompiles).  The
    sources compile in parallel, one hipcc process each, then link."""
    tag = "%d" % os.getpid()
    objs, procs = [], []
    for src in SOURCES:
        obj = os.path.join(PKG_DIR, "_%s.%s.o" % (src.replace(".", "_"), tag))
        cmd = [hipcc()] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    try:
        outs = []
        for cmd, proc in procs:
            out, _ = proc.communicate()
            out = _quiet(out)
            if proc.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + out)
            outs.append(out)
        tmp = LIB_PATH + ".tmp" + tag
        cmd = [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp] + objs
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc link failed:\n" + " ".join(cmd) + "\n" + _quiet(res.stdout))
        if verbose:
            for out in outs + [_quiet(res.stdout)]:
                if out.strip():
                    print(out)
        os.replace(tmp, LIB_PATH)
    finally:
        for obj in objs:
            if os.path.exists(obj):
                os.remove(obj)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
