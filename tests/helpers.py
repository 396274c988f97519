"""Shared plumbing of the GPU parity tests: moving seeded inputs to the host,
running the oracle on chosen rows, and the attention tolerance check.

Tolerance for attention outputs (float): max |out - ref| <= 2e-3 over every
element, and per (row, head) ||out - ref||_2 / max(||ref||_2, 1e-6) <= 1e-3,
against the fp64 oracle that consumes the same dequantised values.  lse is
checked to 1e-4 absolute (the only inexact steps before it are the fp32
accumulation of exact fp16 products and the fp32 exp/log).  Integer outputs
(codes, scales, indices) must match exactly.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

ATOL = 2e-3
RTOL_L2 = 1e-3
LSE_ATOL = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16/int16 tensor -> numpy uint16 bit patterns."""
    return np_(t.contiguous().view(torch.int16)).view(np.uint16)


def kv_host(kv: torch.Tensor):
    """(array, dtype tag) of raw KV rows for the oracle quantiser."""
    if kv.dtype == torch.float32:
        return np_(kv), "f32"
    return bits16(kv), "bf16"


def oracle_quantize(kv: torch.Tensor):
    x, tag = kv_host(kv)
    rows, D = x.shape
    codes = np.zeros((rows, D // 2), np.uint8)
    scales = np.zeros((rows, D // 16), np.uint8)
    oracle.quantize_append(x, tag, np.arange(rows, dtype=np.int64), codes, scales)
    return codes, scales


def check_attn(out, ref, lse=None, lse_ref=None, what=""):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    err = np.abs(out - ref)
    num = np.linalg.norm(out - ref, axis=-1)
    den = np.maximum(np.linalg.norm(ref, axis=-1), 1e-6)
    rel = num / den
    log(f"  {what}: max_abs={err.max():.3e} max_rel_l2={rel.max():.3e}")
    assert err.max() <= ATOL, f"{what}: max abs error {err.max():.3e} > {ATOL}"
    assert rel.max() <= RTOL_L2, f"{what}: rel L2 error {rel.max():.3e} > {RTOL_L2}"
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        lse_ref = np.asarray(lse_ref, np.float64)
        inf_a, inf_b = np.isneginf(lse), np.isneginf(lse_ref)
        assert np.array_equal(inf_a, inf_b), f"{what}: -inf lse pattern differs"
        fin = ~inf_a
        if fin.any():
            d = np.abs(lse[fin] - lse_ref[fin]).max()
            assert d <= LSE_ATOL, f"{what}: lse error {d:.3e}"


def oracle_attn_rows(wl, topk_by_row, layer, rows, W, scale):
    """Oracle attention for the given rows of one layer.

    Only the entries a row attends to are quantised by the oracle (from the raw
    KV), which keeps full-size checks cheap; the key set, and so the result, is
    the same as with the whole cache.  topk_by_row: {row: oracle index list}.
    Returns {row: (out [H, D], lse [H])}."""
    res = {}
    seq_start = np_(wl.seq_start)
    row_seq = np_(wl.row_seq)
    row_len = np_(wl.row_len)
    swa_start = np_(wl.swa_row_start)
    swa_len = np_(wl.swa_len)
    for r in rows:
        idx = np.asarray(topk_by_row[r], np.int64)
        n = int(row_len[r])
        sel = idx[(idx >= 0) & (idx < n)]
        base = int(seq_start[row_seq[r]])
        kv = wl.kv_raw[torch.as_tensor(base + sel, device=wl.kv_raw.device)] if len(sel) else \
            wl.kv_raw[:0]
        codes, scales = oracle_quantize(kv) if len(sel) else (np.zeros((1, wl.cfg.D // 2), np.uint8),
                                                             np.zeros((1, wl.cfg.D // 16), np.uint8))
        K = len(idx)
        local = np.full((1, max(K, 1)), -1, np.int32)
        local[0, :len(sel)] = np.arange(len(sel))
        ns = int(min(max(swa_len[r], 0), W))
        s0 = int(swa_start[r])
        swa = np_(wl.swa[layer][s0:s0 + max(ns, 1)]) if W > 0 else np.zeros((1, wl.cfg.D), np.uint8)
        q = bits16(wl.q[layer][r:r + 1])
        out, lse = oracle.sparse_attn(q, codes, scales, np.zeros(1, np.int64), np.zeros(1, np.int32),
                                      np.array([max(len(sel), 0)], np.int32), local, swa,
                                      np.zeros(1, np.int64), np.array([ns], np.int32), W, scale)
        res[r] = (out[0], lse[0])
    return res


def oracle_index_rows(wl, layer_full, rows, K, P):
    """Oracle Full-mode Top-K and pool for chosen rows (the rows' own data)."""
    qI = np_(wl.qI[layer_full])[rows]
    w = np_(wl.w[layer_full])[rows]
    row_seq = np_(wl.row_seq)[rows]
    row_len = np_(wl.row_len)[rows]
    seqs = sorted(set(int(s) for s in row_seq))
    seq_start = np_(wl.seq_start)
    lengths = wl.lengths
    # pack just the needed sequences' keys
    parts, new_start, remap = [], [], {}
    off = 0
    for s in seqs:
        a, n = int(seq_start[s]), int(lengths[s])
        parts.append(np_(wl.ikeys[a:a + n]))
        remap[s] = len(new_start)
        new_start.append(off)
        off += n
    keys = np.concatenate(parts) if parts else np.zeros((0, wl.cfg.Di), np.uint8)
    rs = np.array([remap[int(s)] for s in row_seq], np.int32)
    topk, pool = oracle.index_full(qI, w, keys, np.array(new_start, np.int64), rs, row_len,
                                   int(row_len.max()), K, P)
    return topk, pool, (keys, np.array(new_start, np.int64), rs, row_len)


def oracle_reindex_rows(wl, layer, rows, packed, pool, K):
    """Oracle Reindex-mode Top-K for the same rows, on the oracle's own pool."""
    keys, starts, rs, row_len = packed
    return oracle.index_reindex(np_(wl.qI[layer])[rows], np_(wl.w[layer])[rows], keys, starts, rs,
                                row_len, pool, K)
