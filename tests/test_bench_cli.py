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


def test_algorithmic_bytes_and_flops_of_the_decode_workloads():
    """Per-unit figures: 128 B per scored entry, 16,384 x 128 B per Reindex
    row-layer, 411,648 B per attention row-layer at D = 512, K = 512, W = 128,
    H = 64; 16,384 FP8 FLOP per scored entry and 2 x 2 x 64 x 512 per key."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    cfg = workloads.CONFIGS[2]
    n = np.full(32, 65536, np.int64)
    b = bench.algorithmic_bytes(cfg, n, 32, n)
    assert b["a5_per_layer"] == 32 * 411648
    assert b["a4_per_layer"] == 32 * (16384 * 128 + 64 * 128 + 64 * 4 + 2048 * 4 + 512 * 4)
    assert b["total"] == 735650816
    f = bench.algorithmic_flops(cfg, 32, n)
    assert f["index_full"] == 32 * 65536 * 16384
    assert f["index_reindex"] == 32 * 16384 * 16384
    assert f["sparse_attn"] == 32 * 640 * 4 * 64 * 512
    cfg3 = workloads.CONFIGS[3]
    n3 = np.full(4, 1 << 20, np.int64)
    per_row = 134217728 + 8192 + 256 + 2048 + 8192 + 3 * (2097152 + 8192 + 256 + 8192 + 2048) + 20 * 411648 + 1312
    assert bench.algorithmic_bytes(cfg3, n3, 4, n3)["total"] == 4 * per_row
