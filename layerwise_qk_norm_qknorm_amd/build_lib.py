"""Builds libqknorm.so (the QK-Norm C ABI) and libstreamceil.so (the
benchmark's streaming copy and read kernels) in-tree with hipcc for gfx950.

    python -m layerwise_qk_norm_qknorm_amd.build_lib

Every build recompiles all sources. The libraries are written next to this
file, where the binding (``libqknorm.so``) and bench.py (``libstreamceil.so``)
load them from.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqknorm.so")
CEIL_LIB = os.path.join(PKG, "libstreamceil.so")

SOURCES = ["qknorm_api.cpp", "qknorm_kernels.hip"]
CEIL_SOURCES = ["stream_ceiling.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqknorm.so)")


def command(out, sources=SOURCES):
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # Packed fp32 instructions stay off: the compiler would form them
        # from plain float code, and they are not used anywhere here.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in sources],
        "-o", out,
    ]


def _build_one(lib, sources, verbose):
    tmp = lib + ".tmp"
    cmd = command(tmp, sources)
    if verbose:
        print("[build] " + " ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def build(verbose=True):
    """Compiles both libraries; returns the path of libqknorm.so."""
    _build_one(CEIL_LIB, CEIL_SOURCES, verbose)
    return _build_one(LIB, SOURCES, verbose)


if __name__ == "__main__":
    print(build())
