"""Build libfva.so in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfva.so")
SOURCES = ["fva_route.hip", "fva_static.hip", "fva_sasa.hip", "fva_attn.hip", "fva_api.cpp"]
HEADERS = ["fva_dev.h", "fva_kernels.h"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source extras.  The attention kernels never test for NaN (their inputs
# are finite by contract, and -inf marks excluded keys), so max/min need no
# NaN canonicalisation there; the router keeps IEEE NaN handling because it
# detects non-finite score rows.
SOURCE_FLAGS = {
    "fva_attn.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
}


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stderr[-8000:])


def build(verbose: bool = False) -> str:
    inc = ["-I", os.path.join(HERE, "..", "include")]
    tag = ".tmp%d" % os.getpid()
    objs = []
    try:
        for src in SOURCES:
            obj = os.path.join(CSRC, src + tag + ".o")
            _run([hipcc()] + HIPCC_FLAGS + SOURCE_FLAGS.get(src, []) + inc +
                 ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
            objs.append(obj)
        tmp = LIB + tag
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(HERE, "..", "include", "fva.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    print(build(verbose=True))
