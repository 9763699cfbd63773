"""Build libkvfp4.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree,
and libkvfp4_yardstick.so (the benchmark's streaming yardsticks, no part of
the library's interface).

    python -m nvfp4_paged_decode_amd.build

Every build recompiles from source.  The libraries land next to this file.
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
LIB = os.path.join(PKG, "libkvfp4.so")
YARDSTICK_LIB = os.path.join(PKG, "libkvfp4_yardstick.so")

SOURCES = ["api.hip", "codec.hip", "decode.hip", "decode_gqa.hip", "decode_gqa_mfma.hip",
           "decode_mla.hip", "order.hip", "rope.hip"]

# gfx950 only.  Packed-fp32 VALU ops are switched off (the host pass warns
# that it does not know the feature; harmless).  No fast-math: the codec
# relies on IEEE fp32/fp64 arithmetic with denormals.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libkvfp4)")


def _compile(sources, out: str, verbose: bool) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *FLAGS, "-I", INCLUDE, "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (res.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    _compile(["yardstick.hip"], YARDSTICK_LIB, verbose)
    return _compile(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
