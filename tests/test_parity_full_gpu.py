"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (one CSA2Step over all layers).  The oracle recomputes a seeded
sample of rows (the whole row: every entry's score, the Top-K, the pool, each
Reindex layer, and attention on sampled layers) and a sample of quantised cache
rows; every sampled integer output must match exactly and every sampled
attention output must meet the tolerance."""
import math

import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as csa2
from sparse_attention_fp4_amd.step import CSA2Step, parent_layers
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


SAMPLES = {
    2: dict(rows=[0, 17, 31], attn_layers=[0, 1, 5, 12, 19]),
    3: dict(rows=[2], attn_layers=[0, 5, 19]),
    4: dict(rows=[0, 1234, 4095], attn_layers=[0]),
    5: dict(rows=None, attn_layers=[0, 10, 16]),
    6: dict(rows=[0, 2047, 4095], attn_layers=[0, 3, 5, 19]),
}


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
    par = parent_layers(modes)
    rows = SAMPLES[cid]["rows"]
    if rows is None:
        lens = wl.lengths
        rng = np.random.default_rng(cfg.seed)
        rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), *rng.choice(len(lens), 2, replace=False).tolist()})

    # quantised cache: a seeded sample of rows
    rng = np.random.default_rng(cfg.seed + 7)
    qrows = np.unique(rng.integers(0, wl.rows_total, 256))
    qrows_t = torch.tensor(qrows, device=DEV)
    rc, rs = oracle_quantize(wl.kv_raw[qrows_t])
    assert np.array_equal(np_(step.codes[qrows_t]), rc), "codes differ"
    assert np.array_equal(np_(step.scales[qrows_t]), rs), "scales differ"
    log("  quantised rows match")

    # Full layer: Top-K and pool of the sampled rows
    log(f"  oracle Full index for rows {rows}")
    rt, rp, packed = oracle_index_rows(wl, 0, rows, cfg.K, cfg.P)
    assert np.array_equal(np_(step.topk[0])[rows], rt), "Full top-k differs"
    assert np.array_equal(np_(step.pool)[rows], rp), "pool differs"
    oracle_topk = {0: rt}
    for l, m in enumerate(modes):
        if m == "R":
            want = oracle_reindex_rows(wl, l, rows, packed, rp, cfg.K)
            assert np.array_equal(np_(step.topk[l])[rows], want), f"Reindex layer {l} differs"
            oracle_topk[l] = want
    log("  index outputs match")

    for l in SAMPLES[cid]["attn_layers"]:
        parent = oracle_topk[par[l]]
        ref = oracle_attn_rows(wl, {r: parent[i] for i, r in enumerate(rows)}, l, rows, cfg.W,
                               1.0 / math.sqrt(cfg.D))
        out = np_(step.out[l])[rows]
        lse = np_(step.lse[l])[rows]
        check_attn(out, np.stack([ref[r][0] for r in rows]), lse, np.stack([ref[r][1] for r in rows]),
                   what=f"config {cid} layer {l}")
    del step, wl
    torch.cuda.empty_cache()
