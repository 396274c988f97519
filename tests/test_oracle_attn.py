"""Pins of the oracle's sparse attention (CPU only).

Checked against closed forms (zero query -> mean of values; one key -> that
key; equal keys -> the key; no selected entries -> attention over the SWA rows
alone), against an independent dense loop when the selection covers every
entry, and against torch's float64 softmax attention (a library routine).
"""
import numpy as np
import torch

import oracle


def e4m3_bytes(vals):
    return torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def make_cache(rng, rows, D):
    x = rng.standard_normal((rows, D)).astype(np.float32)
    codes = np.zeros((rows, D // 2), np.uint8)
    scales = np.zeros((rows, D // 16), np.uint8)
    oracle.quantize_append(x, "f32", np.arange(rows, dtype=np.int64), codes, scales)
    return codes, scales


def call(q, codes, scales, n, idx, swa, swa_len, W, scale=0.125, R=1):
    return oracle.sparse_attn(bits(q), codes, scales, np.zeros(R, np.int64), np.zeros(R, np.int32),
                              np.full(R, n, np.int32), np.asarray(idx, np.int32), swa,
                              np.zeros(R, np.int64), np.full(R, swa_len, np.int32), W, scale)


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(0)
    D, n = 32, 50
    codes, scales = make_cache(rng, n, D)
    vals = oracle.dequant_rows(codes, scales)
    idx = np.array([[3, 7, 11, 20, -1, 49]])
    swa = e4m3_bytes(rng.standard_normal((4, D)))
    q = bf16(np.zeros((1, 2, D)))
    o, lse = call(q, codes, scales, n, idx, swa, 4, 4)
    keys = np.concatenate([vals[[3, 7, 11, 20, 49]],
                           torch.tensor(swa).view(torch.float8_e4m3fn).double().numpy()])
    np.testing.assert_allclose(o[0, 0], keys.mean(0), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(lse[0], np.log(len(keys)), rtol=1e-6)


def test_single_key_returns_it():
    rng = np.random.default_rng(1)
    D = 64
    codes, scales = make_cache(rng, 10, D)
    vals = oracle.dequant_rows(codes, scales)
    q = bf16(rng.standard_normal((1, 3, D)))
    o, _ = call(q, codes, scales, 10, [[-1, 6, -1]], np.zeros((1, D), np.uint8), 0, 0)
    for h in range(3):
        np.testing.assert_array_equal(o[0, h], vals[6].astype(np.float32))


def test_equal_keys_return_the_key():
    D = 16
    x = np.tile(np.linspace(-2, 2, D, dtype=np.float32), (5, 1))
    codes = np.zeros((5, D // 2), np.uint8)
    scales = np.zeros((5, 1), np.uint8)
    oracle.quantize_append(x, "f32", np.arange(5, dtype=np.int64), codes, scales)
    vals = oracle.dequant_rows(codes, scales)
    q = bf16(np.random.default_rng(2).standard_normal((1, 2, D)) * 5)
    o, _ = call(q, codes, scales, 5, [[0, 1, 2, 3, 4]], np.zeros((1, D), np.uint8), 0, 0)
    np.testing.assert_allclose(o[0, 1], vals[0], rtol=1e-6, atol=1e-7)


def test_no_selection_is_swa_only_dense_attention_vs_torch():
    rng = np.random.default_rng(3)
    D, W = 32, 6
    codes, scales = make_cache(rng, 4, D)
    swa = e4m3_bytes(rng.standard_normal((W, D)))
    q = bf16(rng.standard_normal((1, 4, D)))
    o, lse = call(q, codes, scales, 4, [[-1, -1]], swa, W, W, scale=0.3)
    kv = torch.tensor(swa).view(torch.float8_e4m3fn).double()
    qd = q.double()[0]
    p = torch.softmax(0.3 * qd @ kv.T, dim=-1)
    np.testing.assert_allclose(o[0], (p @ kv).numpy(), rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(lse[0], torch.logsumexp(0.3 * qd @ kv.T, -1).numpy(), rtol=1e-6)


def test_empty_key_set():
    D = 16
    codes = np.zeros((2, 8), np.uint8)
    scales = np.zeros((2, 1), np.uint8)
    o, lse = call(bf16(np.ones((1, 1, D))), codes, scales, 2, [[-1, 5]], np.zeros((1, D), np.uint8), 0, 0)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_sparse_equals_dense_when_selection_covers_all_entries():
    rng = np.random.default_rng(4)
    D, H, W = 64, 4, 5
    lens = np.array([9, 17, 3])
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rows = int(lens.sum())
    codes, scales = make_cache(rng, rows, D)
    R = 3
    K = 20                                  # >= every row length
    idx = np.full((R, K), -1, np.int32)
    for r in range(R):
        perm = rng.permutation(lens[r])     # list order must not matter
        idx[r, :lens[r]] = perm
    swa = e4m3_bytes(rng.standard_normal((R * W, D)))
    swa_start = np.arange(R, dtype=np.int64) * W
    swa_len = np.array([5, 0, 3], np.int32)
    q = bf16(rng.standard_normal((R, H, D)))
    o, _ = oracle.sparse_attn(bits(q), codes, scales, starts, np.arange(R, dtype=np.int32),
                              lens.astype(np.int32), idx, swa, swa_start, swa_len, W, 0.125)
    kvv = oracle.dequant_rows(codes, scales)
    swv = torch.tensor(swa).view(torch.float8_e4m3fn).double().numpy()
    dense = oracle.dense_attn(bits(q), kvv, starts, np.arange(R, dtype=np.int32), lens.astype(np.int32),
                              swv, swa_start, swa_len, 0.125)
    np.testing.assert_allclose(o, dense, rtol=1e-6, atol=1e-6)
    # and against torch float64 attention (library routine)
    for r in range(R):
        keys = np.concatenate([kvv[starts[r]:starts[r] + lens[r]], swv[swa_start[r]:swa_start[r] + swa_len[r]]])
        kt = torch.tensor(keys)
        p = torch.softmax(0.125 * q.double()[r] @ kt.T, -1)
        np.testing.assert_allclose(o[r], (p @ kt).numpy(), rtol=1e-6, atol=1e-6)


def test_reuse_layer_attention_uses_inherited_indices():
    """A Reuse layer attends with the parent layer's Top-K list.  Feeding the
    parent's list gives the same output as listing those entries by hand and
    running dense attention over exactly them (torch float64)."""
    rng = np.random.default_rng(5)
    D, H, n = 32, 2, 40
    codes, scales = make_cache(rng, n, D)
    parent_idx = np.array([[1, 5, 9, 33, -1, -1]], np.int32)
    q = bf16(rng.standard_normal((1, H, D)))
    o, _ = call(q, codes, scales, n, parent_idx, np.zeros((1, D), np.uint8), 0, 0, scale=0.2)
    kt = torch.tensor(oracle.dequant_rows(codes, scales)[[1, 5, 9, 33]])
    p = torch.softmax(0.2 * q.double()[0] @ kt.T, -1)
    np.testing.assert_allclose(o[0], (p @ kt).numpy(), rtol=1e-6, atol=1e-6)


def test_out_of_range_indices_contribute_nothing():
    rng = np.random.default_rng(6)
    D = 16
    codes, scales = make_cache(rng, 8, D)
    q = bf16(rng.standard_normal((1, 1, D)))
    a, _ = call(q, codes, scales, 5, [[0, 2, 7, 100, -3]], np.zeros((1, D), np.uint8), 0, 0)
    b, _ = call(q, codes, scales, 5, [[0, 2, -1, -1, -1]], np.zeros((1, D), np.uint8), 0, 0)
    np.testing.assert_array_equal(a, b)


def test_layer_schedule_reuse_links():
    from oracle.step import parents
    modes = list("F" + "UUUU" + "R" + "UUUU" + "R" + "UUUU" + "R" + "UUUU")
    p = parents(modes)
    assert p[0] == 0 and p[1:5] == [0] * 4
    assert p[5] == 5 and p[6:10] == [5] * 4
    assert p[15:] == [15] * 5
    assert parents(list("FRU")) == [0, 1, 1]
