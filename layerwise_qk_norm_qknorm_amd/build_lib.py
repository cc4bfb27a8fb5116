"""Builds libqknorm.so (the QK-Norm C ABI) and libstreamceil.so (the
benchmark's streaming copy and read kernels) in-tree with hipcc for gfx950,
and their timing-only twins libqknorm_clocks.so and libstreamceil_clocks.so
(the same sources with QKNORM_BLOCK_CLOCKS: every row or copy block records
its start and end clocks; loaded only by ``bench.py --timeline``).

    python -m layerwise_qk_norm_qknorm_amd.build_lib

Every build recompiles all sources. The libraries are written next to this
file, where the binding (``libqknorm.so``) and bench.py (the others) load
them from.
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
CLOCKS_LIB = os.path.join(PKG, "libqknorm_clocks.so")
CEIL_CLOCKS_LIB = os.path.join(PKG, "libstreamceil_clocks.so")

SOURCES = ["qknorm_api.cpp", "qknorm_kernels.hip"]
CEIL_SOURCES = ["stream_ceiling.hip"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqknorm.so)")


def command(out, sources=SOURCES, defines=()):
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function", *[f"-D{d}" for d in defines],
        # Packed fp32 instructions stay off: the compiler would form them
        # from plain float code, and they are not used anywhere here.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        *[os.path.join(CSRC, s) for s in sources],
        "-o", out,
    ]


def _start(lib, sources, defines, verbose):
    tmp = lib + ".tmp"
    cmd = command(tmp, sources, defines)
    if verbose:
        print("[build] " + " ".join(cmd), flush=True)
    return lib, tmp, subprocess.Popen(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(job, verbose):
    lib, tmp, proc = job
    _, stderr = proc.communicate()
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed for {os.path.basename(lib)} ({proc.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, lib)
    return lib


def _build_one(lib, sources, verbose, defines=()):
    return _finish(_start(lib, sources, defines, verbose), verbose)


def build(verbose=True):
    """Compiles the four libraries (two hipcc processes at a time); returns
    the path of libqknorm.so."""
    jobs = [(CEIL_LIB, CEIL_SOURCES, ()), (CEIL_CLOCKS_LIB, CEIL_SOURCES, ("QKNORM_BLOCK_CLOCKS",)),
            (CLOCKS_LIB, SOURCES, ("QKNORM_BLOCK_CLOCKS",)), (LIB, SOURCES, ())]
    for a, b in (jobs[:2], jobs[2:]):
        running = [_start(lib, src, defs, verbose) for lib, src, defs in (a, b)]
        for job in running:
            _finish(job, verbose)
    return LIB


if __name__ == "__main__":
    print(build())
