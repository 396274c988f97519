#!/usr/bin/env python3
"""Benchmark of the CSA2 decode step on one MI355X.

A step is one pass of the whole hot path for one batch: the new compressed
entry of every sequence is quantised and appended, the Full layer scores every
entry and selects its Top-K and block pool, each Reindex layer rescores the
pool, and every layer (Full, Reindex and Reuse) runs sparse attention over its
selected entries plus its FP8 sliding window.  Inputs are seeded synthetic
data already resident in HBM.  The step is captured once as a HIP graph and
replayed; `value` is whole-job decode throughput (query rows per second).

Also reported: the algorithmic HBM bytes moved per step and the achieved
fraction of the 8 TB/s peak, a per-call breakdown, a cold-cache step time
(L2 and Infinity Cache flushed before every step), the roofline of the call
that takes most of the step (by measured time x calls per step; sparse
attention, which every layer runs, on the decode workloads) and of the
Full-mode index call, and the CPU oracle timed on a bounded sample of the
same workload on this host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2|3|5|4]
"""
from __future__ import annotations

import argparse
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

# HBM traffic per call measured with rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE per dispatch, scaled by the same counters on a plain 1 GiB device
# copy), keyed by (workload id, call, hash of the kernel source the counters
# were taken on).  Reported as null whenever that source has changed since.
TRAFFIC = {
    # profiles/sparse_attn_decode_64k.md: k_sparse_attn + k_attn_combine per call
    (2, "sparse_attn", "dbb3533f8d62e83a"): 32085009,
    # profiles/index_full_decode_64k.md: k_index_score (Full) + k_select (Full) per call
    (2, "index_full", "3b324613329f3265"): 284831767,
    # profiles/index_reindex_decode_64k.md: k_index_score (Reindex) + k_select (Reindex) per call
    (2, "index_reindex", "3b324613329f3265"): 74539671,
}
CALL_SOURCE = {"sparse_attn": "attn.hip", "index_full": "index.hip", "index_reindex": "index.hip",
               "quantize_append": "quantize.hip"}
CALL_KERNELS = {"sparse_attn": "k_sparse_attn (+ k_attn_combine when key tiles are split)",
                "index_full": "k_index_score + k_select (Full)",
                "index_reindex": "k_index_score + k_select (Reindex)",
                "quantize_append": "k_quantize_append"}


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


def graph_of(fn, reps=1):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm the allocator / code objects outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps, inner=1):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / (reps * inner)


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
        out=step.out[lu], lse=step.lse[lu], workspace=step.workspace)
    for name, fn in calls.items():
        g = graph_of(fn, reps=reps)
        time_graph(g, 2, reps)
        out[name] = time_graph(g, 5, reps) * 1000.0   # us per call
    return out


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
        workspace=step.workspace)
    out = {}
    for name, fn in calls.items():
        g = graph_of(fn, reps=reps)
        time_graph(g, 2, reps)
        out[name] = time_graph(g, 5, reps) * 1000.0
    return out


def cold_step_ms(g, steps):
    """Step time with L2 and Infinity Cache flushed (1 GiB write) before each step."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    times = []
    for _ in range(steps):
        flush.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del flush
    return float(np.median(times))


def copy_check():
    """Plain device copy of 1 GiB (reference kernel for counter scaling) and the
    achieved copy bandwidth."""
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
    return dict(bytes_read=n * 4, bytes_written=n * 4, ms=ms, gbps=2 * n * 4 / ms / 1e6)


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
                sample=f"{rows_done} query-row steps over the {wl.R} rows of the same workload, each a whole step "
                       f"(append + Full + {modes.count('R')} Reindex + {len(modes)} attention layers), "
                       f"{t_total:.1f} s of CPU time with {nthreads} OpenMP threads")


def source_hash(name):
    p = os.path.join(ROOT, "sparse_attention_fp4_amd", "csrc", name)
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


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
    ap.add_argument("--copy-check", action="store_true", help="also time a plain 1 GiB device copy")
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

    cfg = workloads.CONFIGS[args.config]
    log(f"bench: config {cfg.cid} ({cfg.name}) generating inputs")
    wl, step = build(cfg, "cuda")
    R = wl.R
    row_len = wl.row_len.cpu().numpy()
    alg = algorithmic_bytes(cfg, wl.lengths, R, row_len)

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
    g = graph_of(step.run)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    log(f"bench: timing {args.steps} steps")
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    tokens_per_s = R / (ms / 1000.0) if not cfg.prefill_rows else cfg.prefill_rows / (ms / 1000.0)
    step_gbps = alg["total"] / (ms / 1000.0) / 1e9

    breakdown, roofline, index_roofline, reindex_roofline, shares = {}, None, None, None, {}
    if not args.no_breakdown:
        log("bench: per-call timing")
        breakdown = per_call_times(step)
        modes = list(cfg.layers)
        calls_per_step = {"quantize_append": 1, "index_full": modes.count("F"),
                          "index_reindex": modes.count("R"), "sparse_attn": len(modes)}
        call_bytes = {"quantize_append": alg["a1"], "index_full": alg["a2"],
                      "index_reindex": alg["a4_per_layer"], "sparse_attn": alg["a5_per_layer"]}
        shares = {k: breakdown[k] * calls_per_step[k] / 1000.0 / ms for k in breakdown}

        def roof(call):
            us = breakdown[call]
            achieved = call_bytes[call] / (us / 1e6) / 1e9
            tr = TRAFFIC.get((cfg.cid, call, source_hash(CALL_SOURCE[call])))
            return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBPS, 4), traffic=tr,
                        kernel=f"csa2_{call}: {CALL_KERNELS[call]}", us_per_launch=round(us, 2),
                        launches_per_step=calls_per_step[call], share_of_step=round(shares[call], 3),
                        algorithmic_bytes_per_launch=int(call_bytes[call]))
        dominant = max(shares, key=shares.get)
        roofline = roof(dominant)
        index_roofline = roof("index_full")
        if calls_per_step["index_reindex"]:
            reindex_roofline = roof("index_reindex")
    log("bench: cold-cache steps")
    cold_ms = cold_step_ms(g, min(args.steps, 10))
    extra = {}
    if args.page_rows > 0:
        log(f"bench: paged step ({args.page_rows} entries per page)")
        pstep = build_paged(cfg, wl, step, args.page_rows)
        for _ in range(max(args.warmup, 1)):
            pstep.run()
        pg = graph_of(pstep.run)
        time_graph(pg, 2)
        pms = time_graph(pg, args.steps)
        extra["paged"] = {
            "page_rows": args.page_rows,
            "swa": "ring, seeded heads" if pstep.swa_head is not None else "packed",
            "ms_per_step": round(pms, 4),
            "value": round((cfg.prefill_rows or R) / (pms / 1000.0), 1),
            "per_call_us": ({k: round(v, 2) for k, v in per_call_times(pstep).items()}
                            if not args.no_breakdown else {}),
        }
        del pstep, pg
        torch.cuda.empty_cache()
    if args.copy_check:
        extra["copy_check"] = copy_check()

    cpu = None
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cpu = cpu_baseline(cfg, wl)

    D = cfg.D
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8+fp16 mfma, f32 accumulate",
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {
            "workload": (f"{cfg.name}: {R} query rows x {int(row_len.max())} max entries, D={D} FP4 (E2M1 + "
                         f"E4M3/16ch), SWA {cfg.W} FP8, {cfg.H} heads, indexer {cfg.Hi}x{cfg.Di} FP8, "
                         f"Top-{cfg.K}, pool {cfg.P}x8, layers {cfg.layers}"),
            "rows": R, "entries_per_row": int(row_len.max()), "layers": cfg.layers,
        },
        "hbm_gbps_step": round(step_gbps, 1),
        "hbm_frac_step": round(step_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": alg["total"],
        "ms_per_step_cold": round(cold_ms, 4),
        "ms_per_step_eager": round(eager_ms, 3),
        "per_call_us": {k: round(v, 2) for k, v in breakdown.items()},
        "roofline": roofline,
        "roofline_index_full": index_roofline,
        "roofline_index_reindex": reindex_roofline,
        "cpu_baseline": cpu,
    }
    result.update(extra)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
