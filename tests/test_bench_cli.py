"""CPU checks of bench.py's command line: more than one GPU is refused with a
message (this path has no multi-GPU mode), and without a GPU it exits
cleanly instead of falling back to anything."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    p = run("--gpus", "2")
    assert p.returncode == 2
    assert "one GPU only" in p.stderr and p.stdout == ""


def test_no_gpu_exits_without_output():
    import torch
    if torch.cuda.is_available():
        return
    p = run("--steps", "1", "--warmup", "1")
    assert p.returncode == 2 and p.stdout == "" and "needs a GPU" in p.stderr
