#!/usr/bin/env python3
"""Benchmark of the CSA2 decode step on one MI355X.

A step is one pass of the whole hot path for one batch: the new compressed
entry of every sequence is quantised and appended, the Full layer scores every
entry and selects its Top-K and block pool, each Reindex layer rescores the
pool, and every layer (Full, Reindex and Reuse) runs sparse attention over its
selected entries plus its FP8 sliding window.  Inputs are seeded synthetic
data already resident in HBM.  The step is captured once as a HIP graph and
replayed.

Headline (`value`, `ms_per_step`): cold-cache steps -- before each timed step a
1 GiB buffer is written (outside the timed events), which evicts the L2 caches
and the Infinity Cache, so a step cannot re-read the previous step's keys from
cache.  `ms_per_step` is the median of the K timed steps (p10 and p90 beside
it); `value` is whole-job decode throughput, query rows per second (prefill:
chunk tokens per second).  Warm (back-to-back) replays are reported as well.

Also reported: the algorithmic HBM bytes per step and their fraction of the
8 TB/s peak and of a measured device-copy ceiling, a per-call breakdown (HIP
events around graph replays of each call alone), the kernel launches per step
(nodes of the captured graph) and the measured cost of one launch boundary, a
roofline object for the call that takes most of the step and for the index
calls (HBM-bound on decode; matrix-core bound on the prefill chunk), the same
step over a paged copy of the caches, the decode-1M workload (default run), and
the CPU oracle timed on a bounded sample of the same workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|5|4|6|1]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "CSA2 decode tokens/s + achieved HBM GB/s (% of peak) at 64K and 1M KV entries"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp16": 2500.0}   # dense, MI355X

# HBM traffic per call measured with rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE per dispatch, scaled by the same counters on a plain 1 GiB device
# copy), keyed by (workload id, call, hash of the kernel source the counters
# were taken on).  Reported as null whenever that source has changed since.
TRAFFIC = {
    # profiles/sparse_attn_decode_64k.md: k_sparse_attn per call (two key splits merged in the kernel)
    (2, "sparse_attn", "9971ea8daa8c5e19"): 23518208,
    # profiles/sparse_attn_prefill_4096x135k.md: k_sparse_attn per call (four-wave workgroups)
    (4, "sparse_attn", "9971ea8daa8c5e19"): 1562454118,
    # profiles/index_full_decode_64k.md: k_index_score (Full) + k_select (Full) per call
    (2, "index_full", "6efd787f3eacfebd"): 284797850,
    # profiles/index_reindex_decode_64k.md: k_index_score (Reindex) + k_select (Reindex) per call
    (2, "index_reindex", "6efd787f3eacfebd"): 74490163,
    # profiles/index_full_prefill_4096x135k.md: k_index_bmax + k_select (blocks) + k_index_score (rescoring)
    # + k_select (Top-K), twice (two batches of 2,048 rows) per call
    (4, "index_full", "6efd787f3eacfebd"): 1918335795,
}
CALL_SOURCE = {"sparse_attn": "attn.hip", "index_full": "index.hip", "index_reindex": "index.hip",
               "quantize_append": "quantize.hip"}
CALL_KERNELS = {"sparse_attn": "k_sparse_attn (+ k_attn_combine when a row's keys are split more than twice)",
                "index_full": "k_index_score + k_select (Full)",
                "index_reindex": "k_index_score + k_select (Reindex)",
                "quantize_append": "k_quantize_append"}
# csa2_index_full from 1,024 query rows (a prefill chunk), in batches of 2,048 rows
GEMM_FULL_KERNELS = ("k_index_bmax (block maxima, FP8 GEMM) + k_select (pool and candidate blocks) + "
                     "k_index_score (candidates rescored) + k_select (Top-K)")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, lengths, R, row_len):
    """Bytes the method must move per step (per-unit figures of the design):
    a1 2D (bf16 in) + D/2 + D/16 out per appended entry; a2 128 B per visible
    entry plus per-row query, weights and outputs; a4 16,384 x Di gathered key
    bytes plus query, weights, pool and outputs per row-layer; a5 selected FP4
    entries, SWA rows, query, output and index list per row-layer."""
    D, Di, Hi, H, K, P, W = cfg.D, cfg.Di, cfg.Hi, cfg.H, cfg.K, cfg.P, cfg.W
    modes = list(cfg.layers)
    n = np.asarray(row_len, np.int64)
    in_bytes = 2 if cfg.kv_dtype == "bf16" else 4
    appended = cfg.prefill_rows if cfg.prefill_rows else R
    a1 = appended * (D * in_bytes + D // 2 + D // 16)
    a2 = int((n * Di).sum()) + R * (Hi * Di + Hi * 4 + K * 4 + P * 4)
    cand = np.minimum(P * 8, n)
    kfull = np.minimum(K, n)
    a4_one = int((cand * Di).sum()) + R * (Hi * Di + Hi * 4 + P * 4 + K * 4)
    a5_one = int((kfull * (D // 2 + D // 16)).sum()) + R * (W * D + H * D * 2 + H * D * 4 + K * 4)
    nR = sum(1 for m in modes if m == "R")
    total = a1 + a2 + nR * a4_one + len(modes) * a5_one
    return dict(a1=a1, a2=a2, a4_per_layer=a4_one, a5_per_layer=a5_one, total=total)


def algorithmic_flops(cfg, R, row_len):
    """Matrix-core work per call: the indexer takes Hi x Di multiply-adds (FP8)
    per scored entry; attention 2 x H x D multiply-adds (QK^T and PV, fp16) per
    key (selected entries plus the window)."""
    n = np.asarray(row_len, np.int64)
    per_entry = 2 * cfg.Hi * cfg.Di
    return dict(index_full=int(n.sum()) * per_entry,
                index_reindex=int(np.minimum(cfg.P * 8, n).sum()) * per_entry,
                sparse_attn=int((np.minimum(cfg.K, n) + cfg.W).sum()) * 4 * cfg.H * cfg.D,
                quantize_append=0)


def build(cfg, dev):
    import sparse_attention_fp4_amd as csa2
    from sparse_attention_fp4_amd.step import CSA2Step
    wl = workloads.make(cfg, dev)
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=dev)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=dev), codes, scales)
    new_kv = wl.kv_raw[wl.new_rows].contiguous()
    step = CSA2Step(list(cfg.layers), codes=codes, scales=scales, ikeys=wl.ikeys, seq_start=wl.seq_start,
                    row_seq=wl.row_seq, row_len=wl.row_len, max_len=int(wl.row_len.max().item()),
                    new_kv=new_kv, new_rows=wl.new_rows, qI=wl.qI, w=wl.w, q=wl.q, swa=wl.swa,
                    swa_row_start=wl.swa_row_start, swa_len=wl.swa_len, W=cfg.W, K=cfg.K, P=cfg.P,
                    softmax_scale=1.0 / math.sqrt(D))
    return wl, step


def build_paged(cfg, wl, step, page_rows):
    """The same step over a paged copy of the caches: pages of `page_rows`
    entries in shuffled order, and (decode) each row's SWA window stored as a
    ring with a seeded head."""
    from sparse_attention_fp4_amd.step import CSA2Step
    lay = workloads.paged_layout(wl.lengths, page_rows, cfg.seed + 7, device="cuda")
    codes, scales, ikeys = (workloads.to_pages(lay, t) for t in (step.codes, step.scales, step.ikeys))
    new_rows = lay.dst[wl.new_rows] if wl.new_rows is not None else None
    swa, head = wl.swa, None
    if not cfg.prefill_rows and cfg.W > 0:
        g = torch.Generator(device="cuda")
        g.manual_seed(cfg.seed + 8)
        head = torch.randint(0, cfg.W, (wl.R,), generator=g, device="cuda", dtype=torch.int32)
        swa = {l: workloads.swa_ring(t, wl.swa_row_start, cfg.W, head) for l, t in wl.swa.items()}
    return CSA2Step(list(cfg.layers), codes=codes, scales=scales, ikeys=ikeys, seq_start=None,
                    row_seq=wl.row_seq, row_len=wl.row_len, max_len=step.max_len, new_kv=step.new_kv,
                    new_rows=new_rows, qI=wl.qI, w=wl.w, q=wl.q, swa=swa, swa_row_start=wl.swa_row_start,
                    swa_len=wl.swa_len, W=cfg.W, K=cfg.K, P=cfg.P, softmax_scale=step.scale,
                    block_table=lay.block_table, page_rows=page_rows, swa_head=head)


def new_graph(keep=False):
    if keep:
        try:
            return torch.cuda.CUDAGraph(keep_graph=True)
        except TypeError:
            pass
    return torch.cuda.CUDAGraph()


def graph_of(fn, reps=1, keep=False):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm the allocator / code objects outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = new_graph(keep)
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def graph_kernel_nodes(g):
    """(kernel nodes, all nodes) of a captured graph, from the HIP runtime."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        graph = ctypes.c_void_p(g.raw_cuda_graph())
        n = ctypes.c_size_t(0)
        if hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) != 0:
            return None
        nodes = (ctypes.c_void_p * n.value)()
        if hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) != 0:
            return None
        kernels = 0
        for nd in nodes[:n.value]:
            t = ctypes.c_int(-1)
            hip.hipGraphNodeGetType(ctypes.c_void_p(nd), ctypes.byref(t))
            kernels += t.value == 0   # hipGraphNodeTypeKernel
        return kernels, int(n.value)
    except Exception as e:  # noqa: BLE001 - reporting only
        log(f"bench: graph node count unavailable ({e})")
        return None


def time_graph(g, reps, inner=1):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * inner)


def launch_boundary_us(reps=64):
    """Device time per launch of a graph of back-to-back one-thread kernels
    (csa2_paged_rows over a single entry): the fixed cost of one kernel
    boundary inside a graph."""
    import sparse_attention_fp4_amd as csa2
    bt = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    one = torch.zeros(1, dtype=torch.int32, device="cuda")
    ln = torch.ones(1, dtype=torch.int32, device="cuda")
    idx = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    phys = torch.empty(1, 1, dtype=torch.int32, device="cuda")
    g = graph_of(lambda: csa2.csa2_paged_rows(bt, 8, 8, one, ln, idx, phys=phys), reps=reps)
    time_graph(g, 3, reps)
    return time_graph(g, 10, reps) * 1000.0


def per_call_times(step, reps=10):
    """Average device time of each kind of library call, from HIP events around
    graph replays of that call alone (same buffers and sizes as inside the step)."""
    import sparse_attention_fp4_amd as csa2
    out = {}
    l_full = step.modes.index("F")
    if step.paged:
        return paged_call_times(step, reps)
    calls = {
        "quantize_append": lambda: csa2.csa2_quantize_append(step.new_kv, step.new_rows, step.codes, step.scales),
        "index_full": lambda: csa2.csa2_index_full(
            step.qI[l_full], step.w[l_full], step.ikeys, step.seq_start, step.row_seq, step.row_len,
            step.max_len, step.K, step.P, step.block, topk_idx=step.topk[l_full], pool_blocks=step.pool,
            workspace=step.workspace),
    }
    if "R" in step.modes:
        lr = step.modes.index("R")
        calls["index_reindex"] = lambda: csa2.csa2_index_reindex(
            step.qI[lr], step.w[lr], step.ikeys, step.seq_start, step.row_seq, step.row_len, step.pool, step.K,
            step.block, topk_idx=step.topk[lr], workspace=step.workspace)
    lu = len(step.modes) - 1
    calls["sparse_attn"] = lambda: csa2.csa2_sparse_attn(
        step.q[lu], step.codes, step.scales, step.seq_start, step.row_seq, step.row_len,
        step.topk[step.parents[lu]], step.swa[lu], step.swa_row_start, step.swa_len, step.W, step.scale,
        out=step.out[lu], lse=step.lse[lu], workspace=step.attn_workspace)
    for name, fn in calls.items():
        g = graph_of(fn, reps=reps)
        time_graph(g, 2, reps)
        out[name] = time_graph(g, 5, reps) * 1000.0   # us per call
    return out


def fp4mma_times(step, reps=10):
    """csa2_sparse_attn_fp4mma (query-key products on the native FP4 matrix-core
    product where exact) beside csa2_sparse_attn, both on the last layer's
    inputs made exact for the native product: every E4M3 scale byte rounded
    down to its power of two and the two of each 32-channel block made equal,
    the query rounded to E4M3 under one power-of-two scale per head.  (On such
    inputs the two calls agree bit for bit: tests/test_fp4mma_gpu.py.)"""
    import sparse_attention_fp4_amd as csa2
    lu = len(step.modes) - 1
    rows = step.scales.shape[0]
    sc = (step.scales & 0xF8).view(rows, -1, 2)[:, :, :1].expand(-1, -1, 2).reshape(rows, -1).contiguous()
    q = step.q[lu].float()
    m = q.abs().amax(dim=-1, keepdim=True).clamp_min(2.0 ** -100)
    e = ((m.view(torch.int32) >> 23) & 0xFF) - 127 - 7          # 2^e puts the head's largest |q| in [128, 256)
    up = ((e + 127) << 23).view(torch.float32)                    # exact powers of two
    down = ((127 - e) << 23).view(torch.float32)
    qn = ((q * down).to(torch.float8_e4m3fn).float() * up).to(torch.bfloat16)
    cnt = torch.zeros(1, dtype=torch.int32, device=q.device)
    common = (step.seq_start, step.row_seq, step.row_len, step.topk[step.parents[lu]], step.swa[lu],
              step.swa_row_start, step.swa_len, step.W, step.scale)
    out = torch.empty_like(step.out[lu])
    lse = torch.empty_like(step.lse[lu])
    csa2.csa2_sparse_attn_fp4mma(qn, step.codes, sc, *common, out=out, lse=lse, workspace=step.attn_workspace,
                                 native_fragments=cnt)
    torch.cuda.synchronize()
    native = int(cnt.item())
    res = {"inputs": "last layer's, scales rounded down to powers of two shared per 32 channels, "
                     "query rounded to E4M3 under one power-of-two scale per head",
           "native_fragments": native}
    calls = {
        "fp4mma_us": lambda: csa2.csa2_sparse_attn_fp4mma(qn, step.codes, sc, *common, out=out, lse=lse,
                                                          workspace=step.attn_workspace),
        "dequant_us": lambda: csa2.csa2_sparse_attn(qn, step.codes, sc, *common, out=out, lse=lse,
                                                    workspace=step.attn_workspace),
    }
    for name, fn in calls.items():
        g = graph_of(fn, reps=reps)
        time_graph(g, 2, reps)
        res[name] = round(time_graph(g, 5, reps) * 1000.0, 2)
    del sc, qn
    return res


def paged_call_times(step, reps=10):
    """per_call_times for a step in paged mode."""
    import sparse_attention_fp4_amd as csa2
    l_full = step.modes.index("F")
    bt, pr = step.block_table, step.page_rows
    calls = {
        "quantize_append": lambda: csa2.csa2_quantize_append(step.new_kv, step.new_rows, step.codes, step.scales),
        "index_full_paged": lambda: csa2.csa2_index_full_paged(
            step.qI[l_full], step.w[l_full], step.ikeys, bt, pr, step.row_seq, step.row_len, step.max_len, step.K,
            step.P, step.block, topk_idx=step.topk[l_full], pool_blocks=step.pool, topk_rows=step.phys[l_full],
            workspace=step.workspace),
    }
    if "R" in step.modes:
        lr = step.modes.index("R")
        calls["index_reindex_paged"] = lambda: csa2.csa2_index_reindex_paged(
            step.qI[lr], step.w[lr], step.ikeys, bt, pr, step.row_seq, step.row_len, step.pool, step.K, step.block,
            topk_idx=step.topk[lr], topk_rows=step.phys[lr], workspace=step.workspace)
    lu = len(step.modes) - 1
    calls["sparse_attn_phys"] = lambda: csa2.csa2_sparse_attn_phys(
        step.q[lu], step.codes, step.scales, step.phys[step.parents[lu]], step.swa[lu], step.swa_row_start,
        step.swa_len, step.W, step.scale, swa_head=step.swa_head, out=step.out[lu], lse=step.lse[lu],
        workspace=step.attn_workspace)
    out = {}
    for name, fn in calls.items():
        g = graph_of(fn, reps=reps)
        time_graph(g, 2, reps)
        out[name] = time_graph(g, 5, reps) * 1000.0
    return out


class Flusher:
    """Writes 1 GiB before a cold step: more than the L2 caches and the
    256 MB Infinity Cache hold together."""

    def __init__(self):
        self.buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.fill_(1.0)


def timed_steps(g, steps, flush=None):
    """Per-step device times (ms) of `steps` graph replays, each bracketed by
    its own HIP events; with `flush`, the flush runs before each step, outside
    the events.  The whole loop is bracketed by synchronisations."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def copy_check():
    """Plain device copy of 1 GiB (the reference kernel for counter scaling)
    and its achieved bandwidth: the practical HBM ceiling of this device."""
    n = 1 << 28
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del a, b
    torch.cuda.empty_cache()
    return dict(bytes_read=n * 4, bytes_written=n * 4, ms=round(ms, 4), gbps=round(2 * n * 4 / ms / 1e6, 1))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(cfg, wl, budget_s=15.0):
    """The oracle (as it stands) on this host: whole decode steps for a sample of
    query rows, one row at a time, until about budget_s of CPU work is done."""
    import oracle
    import oracle.step
    nthreads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    D = cfg.D
    modes = list(cfg.layers)
    rows_done, t_total = 0, 0.0
    rng = np.random.default_rng(cfg.seed)
    order = rng.permutation(wl.R)
    visits = [int(order[k % wl.R]) for k in range(64 * wl.R)]   # rows repeat until the budget is spent
    for r in visits:
        b = int(wl.row_seq[r].item())
        a = int(wl.seq_start[b].item())
        n = int(wl.row_len[r].item())
        kv = wl.kv_raw[a:a + n]
        bits = kv.float().cpu().numpy() if cfg.kv_dtype == "f32" else \
            kv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        codes = np.zeros((n, D // 2), np.uint8)
        scales = np.zeros((n, D // 16), np.uint8)
        # the cache as it stands before the step (setup, not timed)
        oracle.quantize_append(bits[:-1], "f32" if cfg.kv_dtype == "f32" else "bf16",
                               np.arange(n - 1, dtype=np.int64), codes, scales)
        s0 = int(wl.swa_row_start[r].item())
        inp = dict(qI={l: wl.qI[l][r:r + 1].cpu().numpy() for l in wl.qI},
                   w={l: wl.w[l][r:r + 1].cpu().numpy() for l in wl.w},
                   q_bits={l: wl.q[l][r:r + 1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                           for l in wl.q},
                   swa={l: wl.swa[l][s0:s0 + cfg.W].cpu().numpy() for l in wl.swa},
                   codes=codes, scales=scales, ikeys=wl.ikeys[a:a + n].cpu().numpy(),
                   seq_start=np.zeros(1, np.int64), row_seq=np.zeros(1, np.int32),
                   row_len=np.array([n], np.int32), max_len=n, swa_row_start=np.zeros(1, np.int64),
                   swa_len=np.array([cfg.W], np.int32))
        t0 = time.perf_counter()
        oracle.quantize_append(bits[n - 1:n], "f32" if cfg.kv_dtype == "f32" else "bf16",
                               np.array([n - 1], np.int64), codes, scales)
        oracle.step.decode_step(modes, inp, cfg.K, cfg.P, cfg.W, 1.0 / math.sqrt(D))
        t_total += time.perf_counter() - t0
        rows_done += 1
        log(f"  cpu oracle: row {r} (n={n}) done, {t_total:.1f}s so far")
        if t_total >= budget_s:
            break
    return dict(value=rows_done / t_total, unit="tokens/s", cores=nthreads, kind="oracle",
                cpu_model=cpu_model(),
                sample=f"{rows_done} query-row steps over the {wl.R} rows of the same workload, each a whole step "
                       f"(append + Full + {modes.count('R')} Reindex + {len(modes)} attention layers), "
                       f"{t_total:.1f} s of CPU time with {nthreads} OpenMP threads")


def source_hash(name):
    p = os.path.join(ROOT, "sparse_attention_fp4_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def pct(a, q):
    return round(float(np.percentile(a, q)), 4)


def measure(cfg, args, flusher, copy_gbps, with_paged=True):
    """Build one workload and measure its step: cold (headline) and warm step
    times, the per-call breakdown, launches per step and the rooflines."""
    log(f"bench: config {cfg.cid} ({cfg.name}) generating inputs")
    wl, step = build(cfg, "cuda")
    R = wl.R
    row_len = wl.row_len.cpu().numpy()
    alg = algorithmic_bytes(cfg, wl.lengths, R, row_len)
    flops = algorithmic_flops(cfg, R, row_len)
    prefill = bool(cfg.prefill_rows)
    rows_per_step = cfg.prefill_rows if prefill else R

    log("bench: eager warmup")
    for _ in range(max(args.warmup, 1)):
        step.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        step.run()
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) / 3 * 1000

    log("bench: capturing the step as a HIP graph")
    g = graph_of(step.run, keep=True)
    nodes = graph_kernel_nodes(g)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} cold-cache steps")
    cold = timed_steps(g, args.steps, flusher)
    log(f"bench: timing {args.steps} warm steps")
    warm_ms = time_graph(g, args.steps)
    ms = float(np.median(cold))
    res = {
        "value": round(rows_per_step / (ms / 1000.0), 1),
        "ms_per_step": round(ms, 4),
        "ms_per_step_p10": pct(cold, 10),
        "ms_per_step_p90": pct(cold, 90),
        "timing": "cold cache: 1 GiB written before each step outside its events; median over the timed steps",
        "value_warm": round(rows_per_step / (warm_ms / 1000.0), 1),
        "ms_per_step_warm": round(warm_ms, 4),
        "ms_per_step_eager": round(eager_ms, 3),
        "algorithmic_bytes_per_step": alg["total"],
    }
    step_gbps = alg["total"] / (ms / 1000.0) / 1e9
    res["hbm_gbps_step"] = round(step_gbps, 1)
    res["hbm_frac_step"] = round(step_gbps / HBM_PEAK_GBPS, 4)
    if copy_gbps:
        res["copy_ceiling_frac_step"] = round(step_gbps / copy_gbps, 4)
    if nodes is not None:
        res["launches_per_step"] = nodes[0]
        res["graph_nodes_per_step"] = nodes[1]

    if not args.no_breakdown:
        log("bench: per-call timing")
        breakdown = per_call_times(step)
        modes = list(cfg.layers)
        calls_per_step = {"quantize_append": 1, "index_full": modes.count("F"),
                          "index_reindex": modes.count("R"), "sparse_attn": len(modes)}
        call_bytes = {"quantize_append": alg["a1"], "index_full": alg["a2"],
                      "index_reindex": alg["a4_per_layer"], "sparse_attn": alg["a5_per_layer"]}
        shares = {k: breakdown[k] * calls_per_step[k] / 1000.0 / warm_ms for k in breakdown}

        def roof(call):
            us = breakdown[call]
            tr = TRAFFIC.get((cfg.cid, call, source_hash(CALL_SOURCE[call])))
            label = GEMM_FULL_KERNELS if call == "index_full" and R >= 1024 else CALL_KERNELS[call]
            extra = dict(kernel=f"csa2_{call}: {label}", us_per_launch=round(us, 2),
                         launches_per_step=calls_per_step[call], share_of_warm_step=round(shares[call], 3))
            if prefill and call != "quantize_append":
                # the chunk's rows share one key set: bound by the matrix cores
                dt = "fp16" if call == "sparse_attn" else "fp8"
                achieved = flops[call] / (us / 1e6) / 1e12
                peak = MFMA_PEAK_TFLOPS[dt]
                return dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
                            frac=round(achieved / peak, 4), traffic=tr, dtype=dt,
                            algorithmic_flops_per_launch=int(flops[call]),
                            algorithmic_bytes_per_launch=int(call_bytes[call]), **extra)
            achieved = call_bytes[call] / (us / 1e6) / 1e9
            r = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                     frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=tr,
                     algorithmic_bytes_per_launch=int(call_bytes[call]), **extra)
            if copy_gbps:
                r["copy_ceiling_frac"] = round(achieved / copy_gbps, 4)
            return r

        dominant = max(shares, key=shares.get)
        res["per_call_us"] = {k: round(v, 2) for k, v in breakdown.items()}
        res["roofline"] = roof(dominant)
        res["roofline_index_full"] = roof("index_full")
        if calls_per_step["index_reindex"]:
            res["roofline_index_reindex"] = roof("index_reindex")
        if not prefill:
            res["roofline_sparse_attn"] = roof("sparse_attn")
            log("bench: native-FP4 attention form")
            res["fp4mma"] = fp4mma_times(step)

    if with_paged and args.page_rows > 0:
        log(f"bench: paged step ({args.page_rows} entries per page)")
        pstep = build_paged(cfg, wl, step, args.page_rows)
        for _ in range(max(args.warmup, 1)):
            pstep.run()
        pg = graph_of(pstep.run)
        pg.replay()
        pcold = timed_steps(pg, args.steps, flusher)
        pms = float(np.median(pcold))
        res["paged"] = {
            "page_rows": args.page_rows,
            "swa": "ring, seeded heads" if pstep.swa_head is not None else "packed",
            "ms_per_step": round(pms, 4),
            "value": round(rows_per_step / (pms / 1000.0), 1),
            "ms_per_step_warm": round(time_graph(pg, args.steps), 4),
            "per_call_us": ({k: round(v, 2) for k, v in per_call_times(pstep).items()}
                            if not args.no_breakdown else {}),
        }
        del pstep, pg
    return wl, step, res


def workload_name(cfg, R, row_len):
    return (f"{cfg.name}: {R} query rows x {int(row_len.max())} max entries, D={cfg.D} FP4 (E2M1 + E4M3/16ch), "
            f"SWA {cfg.W} FP8, {cfg.H} heads, indexer {cfg.Hi}x{cfg.Di} FP8, Top-{cfg.K}, pool {cfg.P}x8, "
            f"layers {cfg.layers}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, help="workload: 2 decode 64K (default), 3 decode 1M, "
                                                          "5 ragged 256, 4 prefill chunk (Full layer), "
                                                          "6 prefill chunk (all 20 layers), 1 tiny")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true")
    ap.add_argument("--no-1m", action="store_true", help="skip the decode-1M object of the default run")
    ap.add_argument("--page-rows", type=int, default=64, help="also time the step over a paged copy of the "
                                                               "caches with pages of this many entries (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no multi-GPU "
              "mode: sequences shard across GPUs with no exchange, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import sparse_attention_fp4_amd as csa2
    csa2.lib()

    log("bench: device copy ceiling")
    copy = copy_check()
    boundary = launch_boundary_us()
    flusher = Flusher()

    cfg = workloads.CONFIGS[args.config]
    wl, step, res = measure(cfg, args, flusher, copy["gbps"])
    R = wl.R
    row_len = wl.row_len.cpu().numpy()
    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(cfg, wl)
    del step, wl
    torch.cuda.empty_cache()

    decode_1m = None
    if args.config == 2 and not args.no_1m:
        cfg3 = workloads.CONFIGS[3]
        wl3, step3, r3 = measure(cfg3, args, flusher, copy["gbps"], with_paged=False)
        r3["workload"] = workload_name(cfg3, wl3.R, wl3.row_len.cpu().numpy())
        decode_1m = r3
        del step3, wl3
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": res.pop("value"),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+fp16 mfma, f32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {
            "workload": workload_name(cfg, R, row_len),
            "rows": R, "entries_per_row": int(row_len.max()), "layers": cfg.layers,
        },
    }
    result.update(res)
    if "launches_per_step" in result:
        result["launch_boundary_us"] = round(boundary, 3)
        result["launch_boundaries_us_per_step"] = round(boundary * result["launches_per_step"], 1)
    result["copy_ceiling"] = copy
    result["cpu_baseline"] = cpu
    if decode_1m is not None:
        result["decode_1m"] = decode_1m
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
