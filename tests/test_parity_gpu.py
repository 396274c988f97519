"""GPU parity: every C-ABI entry point against the CPU oracle on seeded
synthetic inputs.  Codes, scales and index lists must match bit for bit;
attention outputs must meet the tolerance in tests/helpers.py.

Sizes: small cases that span several tiles/workgroups with ragged tails and
the degenerate cases (empty rows, fewer entries than K or P*8, all-equal
scores, -1 and out-of-range indices, empty key sets), plus the tiny workload
in full.  The full-size workloads are in test_parity_full_gpu.py.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.step
import sparse_attention_fp4_amd as csa2
from sparse_attention_fp4_amd.step import CSA2Step
import workloads
from helpers import (bits16, check_attn, log, np_, oracle_attn_rows, oracle_index_rows, oracle_quantize,
                     oracle_reindex_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


def gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


# ----------------------------------------------------------------- quantize

def run_quantize(x, dst=None, rows=None):
    T, D = x.shape
    rows = T if rows is None else rows
    dst = torch.arange(T, dtype=torch.int64, device=DEV) if dst is None else dst
    codes = torch.full((rows, D // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, D // 16), 0xCD, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(x, dst, codes, scales)
    torch.cuda.synchronize()
    return np_(codes), np_(scales)


@pytest.mark.parametrize("case", ["f32_normal_d128", "bf16_normal_d512", "bf16_student_outliers_d512"])
def test_quantize_matches_oracle(case):
    log(f"quantize parity: {case}")
    g = gen(11)
    if case == "f32_normal_d128":
        x = torch.randn(4099, 128, generator=g, device=DEV)
    elif case == "bf16_normal_d512":
        x = torch.randn(3001, 512, generator=g, device=DEV).to(torch.bfloat16)
    else:
        cfg = workloads.scaled(workloads.CONFIGS[5], B=2)
        wl = workloads.make(cfg, DEV, layers=[0], lengths=np.array([1500, 1501]))
        x = wl.kv_raw
    c, s = run_quantize(x)
    rc, rs = oracle_quantize(x)
    assert np.array_equal(s, rs), "scales differ"
    assert np.array_equal(c, rc), "codes differ"


def test_quantize_edge_values_and_midpoints():
    """Zeros, -0, tiny and huge values (saturation), and elements exactly on and
    one ulp around every E2M1 midpoint for every scale code."""
    rows = []
    for S in range(1, 0x7F):
        s = oracle.e4m3_value(S)
        for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            m32 = np.float32(mid * s)
            g = np.zeros(16, np.float32)
            g[0] = np.float32(6.0 * s)
            g[1] = np.nextafter(m32, np.float32(0))
            g[2] = m32
            g[3] = np.nextafter(m32, np.float32(1e30))
            g[4] = -m32
            g[5] = -0.0
            rows.append(g)
        # amax exactly on a scale midpoint (tie between two scale codes) and around it
        if S < 0x7E:
            mid = 0.5 * (s + oracle.e4m3_value(S + 1))
            for v in (np.nextafter(np.float32(6 * mid), np.float32(0)), np.float32(6 * mid),
                      np.nextafter(np.float32(6 * mid), np.float32(1e30))):
                g = np.zeros(16, np.float32)
                g[7] = v
                g[8] = -np.float32(v) * np.float32(0.3)
                rows.append(g)
    special = np.zeros((6, 16), np.float32)
    special[1, :] = -0.0
    special[2, 3] = 1e-30
    special[3, 0] = 3e38
    special[3, 1] = -1.0
    special[4, :] = np.float32(6.0 * 448.0)
    special[5, 2] = np.float32(6.0 * 2.0 ** -10)
    x = np.concatenate([np.stack(rows), special])          # [groups, 16]: one group per row
    xt = torch.tensor(x, device=DEV)
    c, s = run_quantize(xt)
    rc, rs = oracle_quantize(xt)
    assert np.array_equal(s, rs) and np.array_equal(c, rc)


def test_quantize_scatter_and_skips_out_of_range_rows():
    g = gen(12)
    x = torch.randn(40, 32, generator=g, device=DEV).to(torch.bfloat16)
    dst = torch.tensor([(7 * i) % 50 for i in range(38)] + [-1, 50], dtype=torch.int64, device=DEV)
    c, s = run_quantize(x, dst, rows=50)
    rc, rs = oracle_quantize(x)
    d = np_(dst)
    for i in range(38):
        assert np.array_equal(c[d[i]], rc[i]) and np.array_equal(s[d[i]], rs[i])
    untouched = sorted(set(range(50)) - set(int(v) for v in d[:38]))
    assert (c[untouched] == 0xAB).all() and (s[untouched] == 0xCD).all()


# ----------------------------------------------------------------- indexer

def small_workload(lengths, Hi=64, Di=128, idx_dist="int3", w_dist="u01_16", layers="FRU", seed=3, D=128, H=16,
                   W=16, kv_dist="normal"):
    cfg = workloads.Config(90 + seed, "small", B=len(lengths), N=None, D=D, W=W, H=H, Hi=Hi, Di=Di, K=0, P=0,
                           idx_dist=idx_dist, w_dist=w_dist, layers=layers, kv_dist=kv_dist)
    return workloads.make(cfg, DEV, lengths=np.array(lengths))


def gpu_index_full(wl, layer, K, P):
    topk, pool = csa2.csa2_index_full(wl.qI[layer], wl.w[layer], wl.ikeys, wl.seq_start, wl.row_seq,
                                      wl.row_len, int(max(wl.lengths.max(), 1)), K, P, want_pool=P > 0)
    torch.cuda.synchronize()
    return np_(topk), (np_(pool) if pool is not None else None)


@pytest.mark.parametrize("name,lengths,Hi,Di,K,P,idx", [
    ("ragged_int3", [1, 7, 100, 1000, 4097, 20001], 64, 128, 512, 2048, "int3"),
    ("ties_alphabet", [30000, 17, 8191, 25000], 64, 128, 512, 2048, "ties"),
    ("p_below_k", [5000, 3333], 64, 128, 100, 10, "int3"),
    ("small_k_p", [3000, 64, 9], 8, 64, 64, 256, "int3"),
    ("hi40_di256", [6000, 2500], 40, 256, 300, 500, "int3"),
    ("hi1_di64", [4096], 1, 64, 64, 256, "int3"),
    ("empty_row", [0, 900], 16, 64, 32, 40, "int3"),
    # more than 4 rounds of 4,096 block maxima (later rounds re-read from memory); K = 2048 gives
    # 16,384 candidates (4 register rounds)
    ("long_k2048", [200000, 140000], 16, 64, 2048, 2048, "int3"),
    ("long_k_above_p", [150000, 9000], 16, 64, 1500, 700, "ties"),
])
def test_index_full_matches_oracle(name, lengths, Hi, Di, K, P, idx):
    log(f"index_full parity: {name}")
    wl = small_workload(lengths, Hi=Hi, Di=Di, idx_dist=idx)
    rows = list(range(len(lengths)))
    topk, pool = gpu_index_full(wl, 0, K, P)
    rt, rp, _ = oracle_index_rows(wl, 0, rows, K, P)
    assert np.array_equal(topk, rt), f"{name}: top-k differs"
    assert np.array_equal(pool, rp), f"{name}: pool differs"


def test_index_full_all_equal_scores_and_no_pool():
    wl = small_workload([5000, 123], Hi=16, Di=64)
    wl.w[0].zero_()                      # every score is 0: ties everywhere
    topk, pool = gpu_index_full(wl, 0, 200, 30)
    rt, rp, _ = oracle_index_rows(wl, 0, [0, 1], 200, 30)
    assert np.array_equal(topk, rt) and np.array_equal(pool, rp)
    assert topk[0].tolist() == list(range(200))
    topk2, none = gpu_index_full(wl, 0, 200, 0)
    assert none is None and np.array_equal(topk2, rt)


def test_index_full_long_row_all_ties_falls_back():
    # a long row (more block maxima than the registers hold) whose scores are all equal: the sampled
    # threshold keeps every block, more than the pre-filter holds, so the full selection runs
    wl = small_workload([150000, 70000], Hi=8, Di=64)
    wl.w[0].zero_()
    topk, pool = gpu_index_full(wl, 0, 300, 2000)
    rt, rp, _ = oracle_index_rows(wl, 0, [0, 1], 300, 2000)
    assert np.array_equal(topk, rt) and np.array_equal(pool, rp)
    assert topk[0].tolist() == list(range(300)) and pool[1].tolist() == list(range(2000))


def test_index_scores_sharing_low_bits_below_their_varying_bits():
    # every score is k[0] of its entry, one of 1.125, 1.375, 1.625, 1.875: their float bits differ only
    # in bits 22..21 and all hold a 1 in bit 20, so the selector's common-bit mask reaches below the
    # bits it resolves; heavy ties leave the lowest ids to decide
    lengths = [5000, 777]
    wl = small_workload(lengths, Hi=16, Di=64)
    rng = np.random.default_rng(17)
    vals = torch.tensor(rng.choice([1.125, 1.375, 1.625, 1.875], size=wl.ikeys.shape[0]), dtype=torch.float32)
    k0 = vals.to(torch.float8_e4m3fn).view(torch.uint8).to(DEV)
    assert torch.equal(k0.cpu().view(torch.float8_e4m3fn).float(), vals)
    wl.ikeys[:, 0] = k0
    for layer in (0, 1):
        wl.w[layer].zero_()
        wl.w[layer][:, 0] = 1.0
        wl.qI[layer].zero_()
        wl.qI[layer][:, 0, 0] = torch.tensor([1.0]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    K, P = 100, 64
    rows = [0, 1]
    topk, pool = gpu_index_full(wl, 0, K, P)
    rt, rp, packed = oracle_index_rows(wl, 0, rows, K, P)
    assert np.array_equal(topk, rt) and np.array_equal(pool, rp)
    want = oracle_reindex_rows(wl, 1, rows, packed, rp, K)
    got = csa2.csa2_index_reindex(wl.qI[1], wl.w[1], wl.ikeys, wl.seq_start, wl.row_seq, wl.row_len,
                                  torch.tensor(rp, device=DEV), K)
    torch.cuda.synchronize()
    assert np.array_equal(np_(got), want)
    # the Top-K holds the largest value's lowest ids first (the ids ascend within the list)
    s0 = np.flatnonzero(vals.numpy()[:lengths[0]] == 1.875)
    assert len(s0) >= K and rt[0].tolist() == s0[:K].tolist()


def many_rows(seq_lengths, rows, Hi, Di, seed=21, idx_dist="int3"):
    """A workload of several sequences with `rows` = [(sequence, visible
    entries)] query rows (as in a prefill chunk), each with its own indexer
    query and weights."""
    wl = small_workload(seq_lengths, Hi=Hi, Di=Di, idx_dist=idx_dist)
    g = gen(seed)
    R = len(rows)
    wl.row_seq = torch.tensor([s for s, _ in rows], dtype=torch.int32, device=DEV)
    wl.row_len = torch.tensor([n for _, n in rows], dtype=torch.int32, device=DEV)
    wl.qI[0] = workloads.to_e4m3_bytes(torch.randint(-3, 4, (R, Hi, Di), generator=g, device=DEV).float())
    wl.w[0] = torch.round(torch.rand(R, Hi, generator=g, device=DEV) * 16.0) / 16.0
    return wl


@pytest.mark.parametrize("case", ["one_sequence_causal", "mixed_sequences"])
def test_index_full_many_rows_matches_oracle(case):
    """Many query rows per call: the causal rows of one sequence (a prefill
    chunk), and rows of several sequences in arbitrary order."""
    log(f"index_full many rows: {case}")
    if case == "one_sequence_causal":
        seq_lengths = [9000]
        rows = [(0, 8000 + i + 1) for i in range(601)]      # row_len <= the sequence's 9,000 entries
    else:
        seq_lengths = [5000, 7777, 300]
        rng = np.random.default_rng(8)
        rows = []
        for i in range(530):
            s = int(rng.integers(0, 3)) if i % 7 else i % 3
            rows.append((s, int(rng.integers(1, seq_lengths[s] + 1))))
    wl = many_rows(seq_lengths, rows, Hi=16, Di=64)
    K, P = 64, 100
    topk, pool = gpu_index_full(wl, 0, K, P)
    check = [0, 1, 2, 3, 4, 5, 6, 7, 250, 301, len(rows) - 2, len(rows) - 1]
    rt, rp, _ = oracle_index_rows(wl, 0, check, K, P)
    assert np.array_equal(topk[check], rt) and np.array_equal(pool[check], rp)


@pytest.mark.parametrize("case", ["one_sequence_two_batches", "mixed_sequences_ties", "hi64_di128", "hi40_di256"])
def test_index_full_gemm_path_matches_oracle(case):
    """From 1,024 rows Full mode takes the prefill path: block maxima from the
    GEMM kernel (each key tile staged once for 8 rows), the pool and the
    candidate blocks from them, the candidates' entries rescored.  Checked
    against the oracle on sampled rows (both batches of 2,048 rows, tile and
    batch edges): one sequence's causal chunk over two key ranges; rows of
    four sequences interleaved (tiles holding rows of other sequences) with
    tied scores; the 64 x 128 indexer shape; 40 heads x 256 dims."""
    log(f"index_full gemm path: {case}")
    rng = np.random.default_rng(31)
    K, P, Hi, Di, idx = 64, 100, 16, 64, "int3"
    if case == "one_sequence_two_batches":
        seq_lengths = [20000]
        rows = [(0, 17000 + i + 1) for i in range(2100)]
    elif case == "mixed_sequences_ties":
        seq_lengths = [5000, 7777, 300, 18000]
        rows = [(3, 17000 + i) for i in range(40)]
        for i in range(1060):
            s = int(rng.integers(0, 4))
            rows.append((s, int(rng.integers(0, seq_lengths[s] + 1))))
        idx = "ties"
    elif case == "hi64_di128":
        seq_lengths = [12000]
        rows = [(0, 10000 + i + 1) for i in range(1030)]
        K, P, Hi, Di = 512, 2048, 64, 128
    else:
        seq_lengths = [9000, 4000]
        rows = [(i % 5 == 0 and 1 or 0, (4000 if i % 5 == 0 else 8000) - i % 700) for i in range(1100)]
        K, P, Hi, Di = 300, 500, 40, 256
    wl = many_rows(seq_lengths, rows, Hi=Hi, Di=Di, idx_dist=idx)
    topk, pool = gpu_index_full(wl, 0, K, P)
    R = len(rows)
    check = sorted({0, 1, 2, 7, 8, 9, 15, 16, R // 2, R - 9, R - 8, R - 1}
                   | ({2047, 2048, 2049} if R > 2049 else set())
                   | set(int(x) for x in rng.choice(R, 8, replace=False)))
    rt, rp, _ = oracle_index_rows(wl, 0, check, K, P)
    assert np.array_equal(topk[check], rt), f"{case}: top-k differs"
    assert np.array_equal(pool[check], rp), f"{case}: pool differs"


@pytest.mark.parametrize("name,lengths,Hi,Di,K,P,idx", [
    ("ragged_int3", [1, 7, 100, 1000, 4097, 20001], 64, 128, 512, 2048, "int3"),
    ("ties_alphabet", [30000, 17, 8191], 64, 128, 512, 2048, "ties"),
    ("small", [3000, 64, 9], 8, 64, 64, 256, "int3"),
    ("k2048_all_pool", [70000, 20000, 5], 16, 64, 2048, 2048, "int3"),
    ("k_above_pool", [40000, 3000], 16, 64, 700, 64, "ties"),
    # 16 rows of full pools: 512 pool positions per scoring workgroup (a few rows take 256, many 1,024)
    ("rows16_full_pools", [17000] * 16, 16, 64, 512, 2048, "int3"),
])
def test_index_reindex_matches_oracle(name, lengths, Hi, Di, K, P, idx):
    log(f"index_reindex parity: {name}")
    wl = small_workload(lengths, Hi=Hi, Di=Di, idx_dist=idx)
    rows = list(range(len(lengths)))
    _, rpool, packed = oracle_index_rows(wl, 0, rows, K, P)
    want = oracle_reindex_rows(wl, 1, rows, packed, rpool, K)
    pool_t = torch.tensor(rpool, device=DEV)
    got = csa2.csa2_index_reindex(wl.qI[1], wl.w[1], wl.ikeys, wl.seq_start, wl.row_seq, wl.row_len, pool_t, K)
    torch.cuda.synchronize()
    assert np.array_equal(np_(got), want)


def test_index_reindex_unsorted_pool_with_invalid_ids():
    wl = small_workload([2000, 500], Hi=16, Di=64)
    rng = np.random.default_rng(5)
    K, P = 50, 40
    pool = np.full((2, P), -1, np.int32)
    for r, n in enumerate([2000, 500]):
        nb = (n + 7) // 8
        ids = rng.choice(nb, 30, replace=False)
        ids[3] = nb + 5                              # out of range: skipped
        pool[r, :30] = ids
        pool[r, 30:35] = -1
        pool[r, 35:] = rng.choice(np.setdiff1d(np.arange(nb), ids), 5, replace=False)
    packed = oracle_index_rows(wl, 0, [0, 1], K, P)[2]
    want = oracle_reindex_rows(wl, 1, [0, 1], packed, pool, K)
    got = csa2.csa2_index_reindex(wl.qI[1], wl.w[1], wl.ikeys, wl.seq_start, wl.row_seq, wl.row_len,
                                  torch.tensor(pool, device=DEV), K)
    torch.cuda.synchronize()
    assert np.array_equal(np_(got), want)


def test_index_reindex_unsorted_pool_all_ties():
    # every score 0: the Top-K is the K lowest visible entry ids of the pool,
    # whatever order the pool lists its blocks in
    wl = small_workload([3000, 700], Hi=16, Di=64)
    wl.w[1].zero_()
    rng = np.random.default_rng(11)
    K, P = 100, 64
    pool = np.full((2, P), -1, np.int32)
    for r, n in enumerate([3000, 700]):
        nb = (n + 7) // 8
        fixed = [nb - 1, 0, nb // 2]                  # the ragged last block, block 0, a middle one
        ids = np.concatenate([fixed, rng.choice(np.setdiff1d(np.arange(nb), fixed), 37, replace=False)])
        pool[r, rng.permutation(P)[:40]] = ids
    packed = oracle_index_rows(wl, 0, [0, 1], K, P)[2]
    want = oracle_reindex_rows(wl, 1, [0, 1], packed, pool, K)
    got = csa2.csa2_index_reindex(wl.qI[1], wl.w[1], wl.ikeys, wl.seq_start, wl.row_seq, wl.row_len,
                                  torch.tensor(pool, device=DEV), K)
    torch.cuda.synchronize()
    got = np_(got)
    assert np.array_equal(got, want)
    for r, n in enumerate([3000, 700]):
        ent = sorted(j for b in pool[r] if b >= 0 for j in range(8 * b, min(8 * b + 8, n)))
        assert got[r].tolist() == ent[:K] + [-1] * max(0, K - len(ent))


# ----------------------------------------------------------------- attention

def run_attn(wl, layer, topk, W, scale):
    out, lse = csa2.csa2_sparse_attn(wl.q[layer], wl.codes_dev, wl.scales_dev, wl.seq_start, wl.row_seq,
                                     wl.row_len, topk, wl.swa[layer], wl.swa_row_start, wl.swa_len, W, scale)
    torch.cuda.synchronize()
    return np_(out), np_(lse)


def with_cache(wl):
    rows, D = wl.kv_raw.shape
    wl.codes_dev = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    wl.scales_dev = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), wl.codes_dev,
                              wl.scales_dev)
    return wl


@pytest.mark.parametrize("name,lengths,D,H,K,W", [
    ("d128_h8_k64_w32_single_row", [4096], 128, 8, 64, 32),
    ("d128_h8_k512_w64_single_row_4_splits", [4096], 128, 8, 512, 64),
    ("d512_h64_rows24_2_splits", [60 + (977 * i) % 20000 for i in range(24)], 512, 64, 512, 128),
    ("d512_h64_rows24_2_splits_one_empty", [5] + [3000 + 11 * i for i in range(23)], 512, 64, 512, 128),
    # two splits at whole rounds of 8 fragments: 33 fragments (24 + 9), 16 (8 + 8), 17 (16 + 1: the second split
    # holds only the SWA fragment), and one head group per row (100 rows x 16 heads)
    ("d512_h64_rows24_2_splits_k512_w8", [700 + (613 * i) % 9000 for i in range(24)], 512, 64, 512, 8),
    ("d512_h64_rows24_2_splits_k256_w0", [700 + (613 * i) % 9000 for i in range(24)], 512, 64, 256, 0),
    ("d512_h64_rows24_2_splits_k256_w16", [700 + (613 * i) % 9000 for i in range(24)], 512, 64, 256, 16),
    ("d512_h16_rows100_2_splits", [400 + (211 * i) % 5000 for i in range(100)], 512, 16, 512, 128),
    ("d512_h64_student_outliers", [9000, 3000, 20000], 512, 64, 512, 128),
    ("d128_h8_student_outliers_nosplit_rows", [500 + 11 * i for i in range(140)], 128, 8, 64, 32),
    ("d512_h64_k512_w128_split", [9000, 700, 30000], 512, 64, 512, 128),
    ("d512_h64_many_rows_nosplit", [300 + 37 * i for i in range(130)], 512, 64, 512, 128),
    ("d512_h64_many_rows_student_outliers", [700 + 31 * i for i in range(130)], 512, 64, 512, 128),
    ("d256_h24_k100_w7", [1000, 77, 5000, 2222], 256, 24, 100, 7),
    ("d128_h3_k33_w0", [500, 40], 128, 3, 33, 0),
    ("d128_h40_k200_w16", [3000, 250, 900], 128, 40, 200, 16),
    ("d256_h64_k300_w64", [5000, 301, 64], 256, 64, 300, 64),
    ("d128_h48_many_rows_64heads_per_group", [150 + 7 * i for i in range(260)], 128, 48, 64, 16),
    ("d256_h40_many_rows_32heads_per_group", [90 + 5 * i for i in range(300)], 256, 40, 40, 24),
    ("d512_h16_k0_swa_only", [100, 100], 512, 16, 0, 128),
])
def test_sparse_attn_matches_oracle(name, lengths, D, H, K, W):
    log(f"sparse_attn parity: {name}")
    wl = with_cache(small_workload(lengths, Hi=8, Di=64, D=D, H=H, W=W, layers="F",
                                   kv_dist="student_t_outliers" if "outliers" in name else "normal"))
    R = len(lengths)
    rng = np.random.default_rng(len(name))
    topk = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        sel = np.sort(rng.choice(n, k, replace=False)) if k else np.array([], np.int64)
        topk[r, :k] = sel
        if K >= 4 and k >= 4:                      # holes and out-of-range ids are skipped
            topk[r, 1] = -1
            topk[r, 2] = n + 3
    if W > 0:
        sl = np_(wl.swa_len)
        sl[0] = W // 2                              # partial window
        if R > 1:
            sl[1] = 0                               # no window
        wl.swa_len = torch.tensor(sl, device=DEV)
    scale = 1.0 / math.sqrt(D)
    out, lse = run_attn(wl, 0, torch.tensor(topk, device=DEV), W, scale)
    ref = oracle_attn_rows(wl, {r: topk[r] for r in range(R)}, 0, list(range(R)), W, scale)
    check_attn(out, np.stack([ref[r][0] for r in range(R)]), lse, np.stack([ref[r][1] for r in range(R)]),
               what=name)


@pytest.mark.parametrize("name,lengths,D,H,K,W,kv", [
    # eight waves, two key splits per row
    ("d512_h64_split_rows", [9000, 3000, 20000], 512, 64, 512, 128, "normal"),
    # eight waves, outliers in the main cache too
    ("d512_h64_student_outliers", [700 + 31 * i for i in range(40)], 512, 64, 512, 128, "student_t_outliers"),
    # four-wave workgroups (520 rows x 4 head groups = 2,080 groups)
    ("d512_h64_four_waves", [300 + (37 * i) % 900 for i in range(520)], 512, 64, 512, 128, "normal"),
])
def test_sparse_attn_large_window_values(name, lengths, D, H, K, W, kv):
    """Window rows with FP8 values of magnitude 8 and above (most bytes of
    24 x N(0,1)), so window fragments take the exact-score path: checked
    against the oracle on every row (or a seeded sample of many rows)."""
    log(f"sparse_attn large window values: {name}")
    wl = with_cache(small_workload(lengths, Hi=8, Di=64, D=D, H=H, W=W, layers="F", kv_dist=kv))
    g = torch.Generator(device=DEV)
    g.manual_seed(len(name))
    wl.swa[0] = workloads.to_e4m3_bytes(24.0 * torch.randn(wl.swa[0].shape, generator=g, device=DEV))
    assert int(((wl.swa[0] & 0x7F) >= 0x50).sum()) > wl.swa[0].numel() // 2   # |v| >= 8 in most bytes
    R = len(lengths)
    rng = np.random.default_rng(len(name))
    topk = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        topk[r, :k] = np.sort(rng.choice(n, k, replace=False))
    scale = 1.0 / math.sqrt(D)
    out, lse = run_attn(wl, 0, torch.tensor(topk, device=DEV), W, scale)
    rows = list(range(R)) if R <= 40 else sorted(set([0, R - 1] + rng.choice(R, 14, replace=False).tolist()))
    ref = oracle_attn_rows(wl, {r: topk[r] for r in rows}, 0, rows, W, scale)
    check_attn(out[rows], np.stack([ref[r][0] for r in rows]), lse[rows], np.stack([ref[r][1] for r in rows]),
               what=name)


@pytest.mark.parametrize("name,D,H,rows,K,W,kv", [
    ("d512_h64_2080_groups", 512, 64, 520, 512, 128, "normal"),
    ("d512_h64_2080_groups_student_outliers", 512, 64, 520, 512, 128, "student_t_outliers"),
    ("d256_h64_32heads_2060_groups_outliers", 256, 64, 1030, 200, 32, "student_t_outliers"),
    ("d128_h64_64heads_2050_groups", 128, 64, 2050, 64, 16, "normal"),
])
def test_sparse_attn_four_wave_workgroups(name, D, H, rows, K, W, kv):
    """Enough (row, head group) pairs for two four-wave workgroups per compute
    unit (at least 2,048): rounds of four fragments, a-parts of exact scores
    formed from the query registers.  All rows are computed; the oracle checks
    a seeded sample of them."""
    log(f"sparse_attn four-wave parity: {name}")
    lengths = [300 + (37 * i) % 900 for i in range(rows)]
    wl = with_cache(small_workload(lengths, Hi=8, Di=64, D=D, H=H, W=W, layers="F", kv_dist=kv))
    rng = np.random.default_rng(rows)
    topk = np.full((rows, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        topk[r, :k] = np.sort(rng.choice(n, k, replace=False))
    scale = 1.0 / math.sqrt(D)
    out, lse = run_attn(wl, 0, torch.tensor(topk, device=DEV), W, scale)
    assert np.isfinite(out).all()
    if kv == "normal":
        # the cache-row form (paged caches) of the same call: same keys in the
        # same order, so the same bits
        base = np_(wl.seq_start)[np_(wl.row_seq)][:, None]
        phys = torch.tensor(np.where(topk >= 0, topk + base, -1).astype(np.int32), device=DEV)
        o2, l2 = csa2.csa2_sparse_attn_phys(wl.q[0], wl.codes_dev, wl.scales_dev, phys, wl.swa[0], wl.swa_row_start,
                                            wl.swa_len, W, scale)
        torch.cuda.synchronize()
        assert np.array_equal(np_(o2), out) and np.array_equal(np_(l2), lse)
    sample = sorted(set([0, rows - 1] + rng.choice(rows, 10, replace=False).tolist()))
    ref = oracle_attn_rows(wl, {r: topk[r] for r in sample}, 0, sample, W, scale)
    check_attn(out[sample], np.stack([ref[r][0] for r in sample]), lse[sample], np.stack([ref[r][1] for r in sample]),
               what=name)


def test_sparse_attn_pair_merge_is_deterministic_and_leaves_its_workspace_zero():
    """Two key splits per row (24 rows x 4 head groups): the second split of a
    pair merges the first's partial.  Two calls on one workspace give
    bit-identical outputs, and the workspace's arrival words end at zero."""
    lengths = [60 + (977 * i) % 20000 for i in range(24)]
    R, D, H, K, W = len(lengths), 512, 64, 512, 128
    wl = with_cache(small_workload(lengths, Hi=8, Di=64, D=D, H=H, W=W, layers="F"))
    rng = np.random.default_rng(5)
    topk = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        topk[r, :k] = np.sort(rng.choice(n, k, replace=False))
    topk = torch.tensor(topk, device=DEV)
    nb = csa2.csa2_sparse_attn_workspace_bytes(R, H, D, K, W)
    assert nb > 1024
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(2):
        out, lse = csa2.csa2_sparse_attn(wl.q[0], wl.codes_dev, wl.scales_dev, wl.seq_start, wl.row_seq,
                                         wl.row_len, topk, wl.swa[0], wl.swa_row_start, wl.swa_len, W,
                                         1.0 / math.sqrt(D), workspace=ws)
        torch.cuda.synchronize()
        outs.append((out.clone(), lse.clone()))
        assert int(ws[:1024].count_nonzero()) == 0
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref = oracle_attn_rows(wl, {r: np_(topk)[r] for r in (0, 17, 23)}, 0, [0, 17, 23], W, 1.0 / math.sqrt(D))
    check_attn(np_(outs[0][0])[[0, 17, 23]], np.stack([ref[r][0] for r in (0, 17, 23)]),
               np_(outs[0][1])[[0, 17, 23]], np.stack([ref[r][1] for r in (0, 17, 23)]), what="pair merge rows")


def test_sparse_attn_empty_key_set():
    wl = with_cache(small_workload([50, 60], Hi=8, Di=64, D=128, H=8, W=0, layers="F"))
    topk = torch.full((2, 16), -1, dtype=torch.int32, device=DEV)
    out, lse = run_attn(wl, 0, topk, 0, 0.1)
    assert (out == 0).all() and np.isneginf(lse).all()


# ----------------------------------------------------------------- whole tiny workload

def test_tiny_workload_step_matches_oracle():
    """Config 1 (N=4096, D=128, 8 heads, 1x64 indexer, Top-64, 256x8 pool,
    Full + Reindex + Reuse) through the same launch sequence as the benchmark."""
    cfg = workloads.CONFIGS[1]
    wl = workloads.make(cfg, DEV)
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), codes, scales)
    new_kv = wl.kv_raw[wl.new_rows].contiguous()
    scale = 1.0 / math.sqrt(D)
    step = CSA2Step(list(cfg.layers), codes=codes, scales=scales, ikeys=wl.ikeys, seq_start=wl.seq_start,
                    row_seq=wl.row_seq, row_len=wl.row_len, max_len=int(wl.lengths.max()), new_kv=new_kv,
                    new_rows=wl.new_rows, qI=wl.qI, w=wl.w, q=wl.q, swa=wl.swa, swa_row_start=wl.swa_row_start,
                    swa_len=wl.swa_len, W=cfg.W, K=cfg.K, P=cfg.P, softmax_scale=scale)
    step.run()
    torch.cuda.synchronize()
    rc, rs = oracle_quantize(wl.kv_raw)
    assert np.array_equal(np_(codes), rc) and np.array_equal(np_(scales), rs)
    inp = dict(qI={l: np_(t) for l, t in wl.qI.items()}, w={l: np_(t) for l, t in wl.w.items()},
               q_bits={l: bits16(t) for l, t in wl.q.items()}, swa={l: np_(t) for l, t in wl.swa.items()},
               codes=rc, scales=rs, ikeys=np_(wl.ikeys), seq_start=np_(wl.seq_start), row_seq=np_(wl.row_seq),
               row_len=np_(wl.row_len), max_len=int(wl.lengths.max()), swa_row_start=np_(wl.swa_row_start),
               swa_len=np_(wl.swa_len))
    topk, pool, outs = oracle.step.decode_step(list(cfg.layers), inp, cfg.K, cfg.P, cfg.W, scale)
    assert np.array_equal(np_(step.pool), pool)
    for l in topk:
        assert np.array_equal(np_(step.topk[l]), topk[l]), f"layer {l} top-k"
    for l in outs:
        check_attn(np_(step.out[l]), outs[l][0], np_(step.lse[l]), outs[l][1], what=f"tiny layer {l}")
