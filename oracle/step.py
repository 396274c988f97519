"""Oracle decode step: the CSA2 layer schedule over the oracle's functions.

Test infrastructure only (see the package docstring).  Follows the three layer
modes of section 一 of the teardown "DeepSeek V4.1 Flash 拆解"
(austincafe.tech): a Full layer runs its own indexer over every entry, keeps
its Top-K and builds the block pool; a Reindex layer rescores only the pool
with its own indexer query and keeps its own Top-K; a Reuse layer attends with
the indices of the layer it reuses.  Reading of the reuse link: a Reuse layer
inherits from the nearest preceding Full or Reindex layer, and every Reindex
layer uses the pool of the (single) Full layer.
"""
from __future__ import annotations

import numpy as np

from . import index_full, index_reindex, sparse_attn


def parents(modes):
    """For each layer, the layer whose Top-K list it attends with."""
    out, last = [], None
    for l, m in enumerate(modes):
        if m in "FR":
            last = l
        if last is None:
            raise ValueError("the first layer must be Full")
        out.append(last)
    return out


def decode_step(modes, inp, K, P, W, softmax_scale, block=8, attn_rows=None, attn_layers=None):
    """inp: dict with numpy arrays: qI[l], w[l] (F/R layers), q_bits[l], swa[l],
    codes, scales, ikeys, seq_start, row_seq, row_len, max_len, swa_row_start,
    swa_len.  Returns (topk per F/R layer, pool, attention outputs per layer).
    attn_rows / attn_layers restrict which attention outputs are computed."""
    topk, pool, outs = {}, None, {}
    par = parents(modes)
    for l, m in enumerate(modes):
        if m == "F":
            topk[l], pool = index_full(inp["qI"][l], inp["w"][l], inp["ikeys"], inp["seq_start"],
                                       inp["row_seq"], inp["row_len"], inp["max_len"], K, P, block)
        elif m == "R":
            topk[l] = index_reindex(inp["qI"][l], inp["w"][l], inp["ikeys"], inp["seq_start"],
                                    inp["row_seq"], inp["row_len"], pool, K, block)
        if attn_layers is not None and l not in attn_layers:
            continue
        outs[l] = sparse_attn(inp["q_bits"][l], inp["codes"], inp["scales"], inp["seq_start"],
                              inp["row_seq"], inp["row_len"], topk[par[l]], inp["swa"][l],
                              inp["swa_row_start"], inp["swa_len"], W, softmax_scale,
                              rows=attn_rows)
    return topk, pool, outs
