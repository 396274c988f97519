"""Pins of the oracle's indexer, Top-K, pool and Reindex (CPU only).

Checked against: brute-force sorting in pure Python on tiny inputs, numpy's
integer matrix product for the single-head case (a library routine), closed
forms (unit queries read a key's component back; weights scale scores
linearly), and the invariants the hierarchical indexer rests on (Top-K lies in
the pool when P >= K; Reindex with the Full layer's own query reproduces
Full's Top-K; pool positions are whole 8-aligned blocks).
"""
import numpy as np
import pytest
import torch

import oracle


def e4m3_bytes(vals):
    return torch.tensor(np.asarray(vals, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def rand_case(rng, R, n_max, Hi, Di, lo=-3, hi=3, ragged=True, alphabet=None):
    lens = rng.integers(1, n_max + 1, R) if ragged else np.full(R, n_max)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    rows = int(lens.sum())
    if alphabet is not None:
        kv = alphabet[rng.integers(0, alphabet.shape[0], rows)]
    else:
        kv = rng.integers(lo, hi + 1, (rows, Di))
    keys = e4m3_bytes(kv)
    q = e4m3_bytes(rng.integers(lo, hi + 1, (R, Hi, Di)))
    w = (np.round(rng.uniform(0, 1, (R, Hi)) * 16) / 16).astype(np.float32)
    return dict(qI=q, w=w, ikeys=keys, seq_start=starts, row_seq=np.arange(R, dtype=np.int32),
                row_len=lens.astype(np.int32), max_len=int(lens.max()), kv=kv)


def brute_topk(scores, K):
    order = sorted(range(len(scores)), key=lambda j: (-scores[j], j))
    sel = sorted(order[:K])
    return sel + [-1] * (K - len(sel))


def test_single_head_scores_match_integer_matmul():
    rng = np.random.default_rng(0)
    c = rand_case(rng, 3, 50, 1, 16, ragged=False)
    c["w"][:] = 1.0
    s = oracle.index_scores(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"], c["row_len"],
                            c["max_len"])
    qv = torch.tensor(c["qI"]).view(torch.float8_e4m3fn).float().numpy().astype(np.int64)
    for r in range(3):
        dots = c["kv"][c["seq_start"][r]:c["seq_start"][r] + 50].astype(np.int64) @ qv[r, 0]
        assert np.array_equal(s[r], np.maximum(dots, 0).astype(np.float32))


def test_unit_query_reads_back_key_component():
    rng = np.random.default_rng(1)
    Di = 8
    kv = rng.integers(-3, 4, (20, Di))
    keys = e4m3_bytes(kv)
    for d in range(Di):
        q = np.zeros((1, 1, Di))
        q[0, 0, d] = 1
        s = oracle.index_scores(e4m3_bytes(q), np.ones((1, 1), np.float32), keys,
                                np.array([0], np.int64), np.array([0], np.int32),
                                np.array([20], np.int32), 20)
        assert np.array_equal(s[0], np.maximum(kv[:, d], 0).astype(np.float32))


def test_scores_linear_in_weights_and_head_permutation_invariant():
    rng = np.random.default_rng(2)
    c = rand_case(rng, 2, 40, 4, 16, ragged=False)
    args = (c["ikeys"], c["seq_start"], c["row_seq"], c["row_len"], c["max_len"])
    s1 = oracle.index_scores(c["qI"], c["w"], *args)
    s2 = oracle.index_scores(c["qI"], c["w"] * 2, *args)
    assert np.array_equal(s2, 2 * s1)
    perm = [2, 0, 3, 1]
    s3 = oracle.index_scores(c["qI"][:, perm], c["w"][:, perm], *args)
    assert np.array_equal(s3, s1)
    # a head whose weight is zero contributes nothing
    w0 = c["w"].copy()
    w0[:, 1] = 0
    q0 = c["qI"].copy()
    q0[:, 1] = e4m3_bytes(rng.integers(-3, 4, (2, 16)))
    assert np.array_equal(oracle.index_scores(q0, w0, *args), oracle.index_scores(c["qI"], w0, *args))


def test_relu_zeroes_negative_heads():
    # one head with q = -k for every key -> dot < 0 -> contributes 0
    Di = 4
    kv = np.array([[1, 2, 0, 1], [3, 0, 1, 1]])
    q = np.stack([-kv[0], kv[0]])[None]
    s = oracle.index_scores(e4m3_bytes(q), np.array([[1.0, 0.5]], np.float32), e4m3_bytes(kv),
                            np.array([0], np.int64), np.array([0], np.int32),
                            np.array([2], np.int32), 2)
    # key0: head0 dot = -6 -> 0; head1 dot = 6 -> 0.5*6 = 3.
    # key1 = (3,0,1,1): head0 dot = -4 -> 0; head1 dot = 4 -> 0.5*4 = 2.
    assert s[0].tolist() == [3.0, 2.0]


@pytest.mark.parametrize("seed", range(6))
def test_full_topk_and_pool_bruteforce_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    alphabet = rng.integers(-1, 2, (5, 8)) if seed % 2 else None
    c = rand_case(rng, 4, 61, 3, 8, lo=-1 if seed % 2 else -3, hi=1 if seed % 2 else 3,
                  alphabet=alphabet)
    for K, P in ((1, 1), (5, 2), (7, 9), (64, 3), (13, 16)):
        topk, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                       c["row_len"], c["max_len"], K, P)
        s = oracle.index_scores(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                c["row_len"], c["max_len"])
        for r in range(4):
            n = int(c["row_len"][r])
            sc = [float(x) for x in s[r, :n]]
            assert topk[r].tolist() == brute_topk(sc, K)
            bm = [max(sc[8 * b:8 * b + 8]) for b in range((n + 7) // 8)]
            assert pool[r].tolist() == brute_topk(bm, P)


def test_all_equal_scores_take_lowest_indices():
    R, n, Di = 1, 37, 4
    keys = e4m3_bytes(np.ones((n, Di)))
    q = e4m3_bytes(np.ones((R, 2, Di)))
    topk, pool = oracle.index_full(q, np.ones((R, 2), np.float32), keys, np.array([0], np.int64),
                                   np.array([0], np.int32), np.array([n], np.int32), n, 10, 3)
    assert topk[0].tolist() == list(range(10))
    assert pool[0].tolist() == [0, 1, 2]


def test_short_rows_pad_with_minus_one():
    rng = np.random.default_rng(4)
    c = rand_case(rng, 1, 5, 2, 8, ragged=False)
    topk, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                   c["row_len"], 5, 8, 4)
    assert topk[0].tolist() == [0, 1, 2, 3, 4, -1, -1, -1]
    assert pool[0].tolist() == [0, -1, -1, -1]
    # a row with no visible entries
    topk, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                   np.array([0], np.int32), 5, 3, 2)
    assert topk[0].tolist() == [-1, -1, -1] and pool[0].tolist() == [-1, -1]


@pytest.mark.parametrize("ties", [False, True])
def test_topk_inside_pool_when_p_ge_k(ties):
    rng = np.random.default_rng(7 + ties)
    alphabet = rng.integers(-1, 2, (4, 16)) if ties else None
    c = rand_case(rng, 6, 3000, 4, 16, lo=-1 if ties else -3, hi=1 if ties else 3, alphabet=alphabet)
    for K, P in ((16, 16), (64, 100), (200, 200)):
        topk, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                       c["row_len"], c["max_len"], K, P)
        for r in range(6):
            blocks = set(int(b) for b in pool[r] if b >= 0)
            for j in topk[r]:
                if j >= 0:
                    assert int(j) // 8 in blocks


def test_pool_positions_are_whole_aligned_blocks():
    rng = np.random.default_rng(8)
    c = rand_case(rng, 3, 999, 2, 8)
    _, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                c["row_len"], c["max_len"], 16, 20)
    for r in range(3):
        n = int(c["row_len"][r])
        ids = [int(b) for b in pool[r] if b >= 0]
        assert ids == sorted(set(ids))
        assert all(0 <= b < (n + 7) // 8 for b in ids)
        assert len(ids) == min(20, (n + 7) // 8)


@pytest.mark.parametrize("ties", [False, True])
def test_reindex_with_own_full_query_reproduces_full_topk(ties):
    rng = np.random.default_rng(9 + ties)
    alphabet = rng.integers(-1, 2, (6, 16)) if ties else None
    c = rand_case(rng, 5, 2500, 4, 16, lo=-1 if ties else -3, hi=1 if ties else 3, alphabet=alphabet)
    K, P = 40, 48
    topk, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                   c["row_len"], c["max_len"], K, P)
    re = oracle.index_reindex(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                              c["row_len"], pool, K)
    assert np.array_equal(re, topk)


def test_reindex_bruteforce_over_pool_positions():
    rng = np.random.default_rng(12)
    c = rand_case(rng, 4, 300, 3, 8)
    K, P = 10, 6
    _, pool = oracle.index_full(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                                c["row_len"], c["max_len"], K, P)
    q2 = e4m3_bytes(rng.integers(-3, 4, c["qI"].shape))
    w2 = (np.round(rng.uniform(0, 1, c["w"].shape) * 16) / 16).astype(np.float32)
    re = oracle.index_reindex(q2, w2, c["ikeys"], c["seq_start"], c["row_seq"], c["row_len"], pool, K)
    s2 = oracle.index_scores(q2, w2, c["ikeys"], c["seq_start"], c["row_seq"], c["row_len"],
                             c["max_len"])
    for r in range(4):
        n = int(c["row_len"][r])
        cand = [8 * b + t for b in pool[r] if b >= 0 for t in range(8) if 8 * b + t < n]
        order = sorted(cand, key=lambda j: (-float(s2[r, j]), j))
        want = sorted(order[:K])
        assert re[r].tolist() == want + [-1] * (K - len(want))


def test_reindex_ignores_minus_one_and_out_of_range_pool_ids():
    rng = np.random.default_rng(13)
    c = rand_case(rng, 1, 40, 2, 8, ragged=False)
    pool = np.array([[-1, 2, 99, 0]], np.int32)
    re = oracle.index_reindex(c["qI"], c["w"], c["ikeys"], c["seq_start"], c["row_seq"],
                              c["row_len"], pool, 16)
    got = [j for j in re[0] if j >= 0]
    assert got == sorted(list(range(0, 8)) + list(range(16, 24)))
