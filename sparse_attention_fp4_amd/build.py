"""Build the CSA2 HIP library (libcsa2.so) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa2.so")
# the same sources with device-side range checks (-DCSA2_DEBUG): every call
# synchronises and reports skipped out-of-range values as CSA2_ERR_DEVICE_CHECK
LIB_DEBUG = os.path.join(HERE, "libcsa2_debug.so")
SOURCES = ["status.hip", "quantize.hip", "index.hip", "attn.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def _compile(out: str, extra, verbose: bool) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile libcsa2.so and (debug=True) libcsa2_debug.so; returns the release path."""
    _compile(LIB, [], verbose)
    if debug:
        _compile(LIB_DEBUG, ["-DCSA2_DEBUG"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
