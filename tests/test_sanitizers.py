"""AddressSanitizer + UndefinedBehaviorSanitizer over the host code, on the CPU.

* The oracle (oracle/csa2_oracle.c) is compiled with gcc and the sanitizers
  and driven through every entry point on inputs that reach its edge paths
  (tests/sanitize/oracle_driver.c).
* The library's host side (argument validation, workspace queries, status
  strings) is compiled with hipcc with the sanitizers on the host code only
  (each -fsanitize= behind -Xarch_host; the device code is built as usual) and
  driven with arguments that fail every check (tests/sanitize/abi_driver.cpp);
  no call reaches a kernel launch.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), so a
zero exit status means a clean run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
OUT = os.path.join(ROOT, "build", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_fp4_amd", "csrc")


def run(cmd, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    p = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    assert p.returncode == 0, f"{' '.join(cmd)}\n--- stdout\n{p.stdout}\n--- stderr\n{p.stderr[-4000:]}"
    return p.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_driver")
    run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fopenmp", "-o", exe, os.path.join(ROOT, "oracle", "csa2_oracle.c"), os.path.join(HERE, "oracle_driver.c"),
         "-lm"])
    out = run([exe], {"ASAN_OPTIONS": "detect_leaks=1", "OMP_NUM_THREADS": "4"})
    assert "oracle ok" in out


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not found")
def test_library_host_validation_under_asan_ubsan():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "abi_driver")
    srcs = [os.path.join(CSRC, s) for s in ("status.hip", "quantize.hip", "index.hip", "attn.hip")]
    run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-o", exe, os.path.join(HERE, "abi_driver.cpp"), *srcs])
    # the HIP runtime's own allocations at load time are not this code's: no leak check
    out = run([exe], {"ASAN_OPTIONS": "detect_leaks=0"})
    assert "abi ok" in out
