"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one CSA2Step over all layers).

The oracle recomputes, for every query row of the decode workloads (decode-64K,
decode-1M, the ragged batch) and for 64 seeded rows of the prefill chunk, the
whole index path: every entry's score, the Top-K, the block pool and each
Reindex layer's Top-K on the oracle's own pool.  Attention is checked on seeded
(row, layer) pairs, each with the Top-K list the oracle's own layer schedule
(`oracle.step.parents`) assigns to that layer, so a wrong inheritance link in
the library's schedule fails here.  Integer outputs must match exactly;
attention outputs must meet the tolerance of tests/helpers.py.  A sample of
quantised cache rows is checked bit for bit as well."""
import math

import numpy as np
import pytest
import torch

import oracle.step
import sparse_attention_fp4_amd as csa2
from sparse_attention_fp4_amd.step import CSA2Step
import workloads
from helpers import (check_attn, log, np_, oracle_attn_rows, oracle_index_rows, oracle_quantize,
                     oracle_reindex_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def build_step(cfg, wl):
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), codes, scales)
    new_kv = wl.kv_raw[wl.new_rows].contiguous()
    step = CSA2Step(list(cfg.layers), codes=codes, scales=scales, ikeys=wl.ikeys, seq_start=wl.seq_start,
                    row_seq=wl.row_seq, row_len=wl.row_len, max_len=int(np_(wl.row_len).max()), new_kv=new_kv,
                    new_rows=wl.new_rows, qI=wl.qI, w=wl.w, q=wl.q, swa=wl.swa, swa_row_start=wl.swa_row_start,
                    swa_len=wl.swa_len, W=cfg.W, K=cfg.K, P=cfg.P, softmax_scale=1.0 / math.sqrt(D))
    return step


# index rows: "all" or a count of seeded rows (always including the first and
# the last); attention: number of seeded (row, layer) pairs, always including
# the first and last row, the Full layer, a Reindex layer, the last layer and
# (ragged batch) the shortest and longest rows.
PLAN = {
    2: dict(index_rows="all", attn_pairs=16),
    3: dict(index_rows="all", attn_pairs=8),
    5: dict(index_rows="all", attn_pairs=16),
    4: dict(index_rows=64, attn_pairs=16),
    6: dict(index_rows=16, attn_pairs=16),
}


def index_rows_of(cfg, wl, spec):
    R = wl.R
    if spec == "all":
        return list(range(R))
    rng = np.random.default_rng(cfg.seed + 11)
    pick = set(rng.choice(R, size=min(spec, R) - 2, replace=False).tolist()) | {0, R - 1}
    return sorted(pick)[:spec] if len(pick) > spec else sorted(pick)


def attn_pairs_of(cfg, wl, rows, npairs):
    modes = list(cfg.layers)
    L = len(modes)
    rng = np.random.default_rng(cfg.seed + 13)
    first_r = modes.index("R") if "R" in modes else 0
    pairs = {(rows[0], 0), (rows[-1], L - 1), (rows[len(rows) // 2], first_r)}
    if cfg.N is None:
        lens = wl.lengths[np_(wl.row_seq)]
        pairs |= {(int(np.argmin(lens)), int(rng.integers(0, L))), (int(np.argmax(lens)), int(rng.integers(0, L)))}
    while len(pairs) < npairs:
        pairs.add((int(rows[rng.integers(0, len(rows))]), int(rng.integers(0, L))))
    return sorted(pairs)


@pytest.mark.parametrize("cid", [2, 5, 3, 4, 6])
def test_full_size_workload(cid):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = workloads.CONFIGS[cid]
    log(f"full-size parity: config {cid} ({cfg.name}) generating inputs")
    wl = workloads.make(cfg, DEV)
    step = build_step(cfg, wl)
    log(f"  running the step (R={wl.R})")
    step.run()
    torch.cuda.synchronize()
    modes = list(cfg.layers)
    par = oracle.step.parents(modes)   # the oracle's own schedule, not the library's
    rows = index_rows_of(cfg, wl, PLAN[cid]["index_rows"])

    # quantised cache: a seeded sample of rows
    rng = np.random.default_rng(cfg.seed + 7)
    qrows = np.unique(rng.integers(0, wl.rows_total, 256))
    qrows_t = torch.tensor(qrows, device=DEV)
    rc, rs = oracle_quantize(wl.kv_raw[qrows_t])
    assert np.array_equal(np_(step.codes[qrows_t]), rc), "codes differ"
    assert np.array_equal(np_(step.scales[qrows_t]), rs), "scales differ"
    log("  quantised rows match")

    # Full layer: Top-K and pool of every checked row
    log(f"  oracle Full index for {len(rows)} rows")
    rt, rp, packed = oracle_index_rows(wl, 0, rows, cfg.K, cfg.P)
    got_t, got_p = np_(step.topk[0])[rows], np_(step.pool)[rows]
    bad = [rows[i] for i in range(len(rows)) if not np.array_equal(got_t[i], rt[i])]
    assert not bad, f"Full top-k differs on rows {bad[:8]}"
    bad = [rows[i] for i in range(len(rows)) if not np.array_equal(got_p[i], rp[i])]
    assert not bad, f"pool differs on rows {bad[:8]}"
    oracle_topk = {0: rt}
    for l, m in enumerate(modes):
        if m == "R":
            log(f"  oracle Reindex layer {l} for {len(rows)} rows")
            want = oracle_reindex_rows(wl, l, rows, packed, rp, cfg.K)
            got = np_(step.topk[l])[rows]
            bad = [rows[i] for i in range(len(rows)) if not np.array_equal(got[i], want[i])]
            assert not bad, f"Reindex layer {l} differs on rows {bad[:8]}"
            oracle_topk[l] = want
    log("  index outputs match")

    pos = {r: i for i, r in enumerate(rows)}
    pairs = attn_pairs_of(cfg, wl, rows, PLAN[cid]["attn_pairs"])
    missing = sorted({r for r, _ in pairs if r not in pos})
    if missing:   # rows picked only for attention (ragged extremes): oracle index lists for them too
        mt, mp, mpacked = oracle_index_rows(wl, 0, missing, cfg.K, cfg.P)
        extra = {0: mt}
        for l, m in enumerate(modes):
            if m == "R":
                extra[l] = oracle_reindex_rows(wl, l, missing, mpacked, mp, cfg.K)
    by_layer = {}
    for r, l in pairs:
        by_layer.setdefault(l, []).append(r)
    for l, rs_l in sorted(by_layer.items()):
        lists = {r: (oracle_topk[par[l]][pos[r]] if r in pos else extra[par[l]][missing.index(r)]) for r in rs_l}
        ref = oracle_attn_rows(wl, lists, l, rs_l, cfg.W, 1.0 / math.sqrt(cfg.D))
        out = np_(step.out[l])[rs_l]
        lse = np_(step.lse[l])[rs_l]
        check_attn(out, np.stack([ref[r][0] for r in rs_l]), lse, np.stack([ref[r][1] for r in rs_l]),
                   what=f"config {cid} layer {l} rows {rs_l}")
    log(f"  attention matches on {len(pairs)} (row, layer) pairs")
    del step, wl
    torch.cuda.empty_cache()
