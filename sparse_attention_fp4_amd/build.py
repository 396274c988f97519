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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# Per-source flags.  attn.hip keeps matrix-core operands and accumulators in
# ordinary VGPRs: its kernels run two waves per SIMD, and at that occupancy the
# compiler would otherwise split the 256 registers evenly between VGPRs and
# AGPRs, which its working set does not fit.
SOURCE_FLAGS = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(out: str, extra, verbose: bool) -> str:
    """Compile every source to its own object (in parallel), then link."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    objs = [f"{out}.{os.path.splitext(s)[0]}.o" for s in SOURCES]

    def run(cmd):
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)

    cmds = [[hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(s, []), *extra, "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    try:
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            for f in [ex.submit(run, c) for c in cmds]:
                f.result()
        run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return out


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile libcsa2.so and (debug=True) libcsa2_debug.so; returns the release path."""
    _compile(LIB, [], verbose)
    if debug:
        _compile(LIB_DEBUG, ["-DCSA2_DEBUG"], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
