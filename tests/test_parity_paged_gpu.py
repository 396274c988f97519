"""GPU parity of the paged-cache calls.

Each case scatters the packed cache of a small workload over shuffled pages
(the rest of the paged cache holds finite junk that must never be read) and
checks:
  * csa2_index_full_paged / csa2_index_reindex_paged against the oracle, bit
    for bit, when every page is mapped, and the cache rows they also write
    against the block-table formula;
  * with unmapped pages (table value -1, or a page past the cache), against the
    selection rule applied by brute force to the oracle's scores with the
    unmapped entries removed;
  * csa2_paged_rows against the block-table formula, bit for bit;
  * csa2_sparse_attn_phys against csa2_sparse_attn on the packed cache (bit
    for bit: the same keys in the same order) and against the oracle, with
    the SWA window stored as a rotated ring.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.step
import sparse_attention_fp4_amd as csa2
import workloads
from helpers import check_attn, log, np_, oracle_attn_rows, oracle_index_rows, oracle_reindex_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


def small_workload(lengths, Hi=16, Di=64, idx_dist="int3", D=128, H=8, W=16, seed=7, kv_dist="normal"):
    cfg = workloads.Config(80 + seed, "small", B=len(lengths), N=None, D=D, W=W, H=H, Hi=Hi, Di=Di, K=0, P=0,
                           idx_dist=idx_dist, w_dist="u01_16", layers="FR", kv_dist=kv_dist)
    return workloads.make(cfg, DEV, lengths=np.array(lengths))


class Pages:
    """Block table over shuffled pages for the sequences of a workload.

    holes: {(seq, page): value} overrides table entries after the layout is
    made (-1, or a page id past the cache): those entries are not visible."""

    def __init__(self, lengths, page_rows, seed, spare=3, holes=None):
        rng = np.random.default_rng(seed)
        self.pr = page_rows
        self.lengths = np.asarray(lengths, np.int64)
        npages = [(int(n) + page_rows - 1) // page_rows for n in lengths]
        self.max_pages = max(max(npages), 1) + 1            # a spare column stays unmapped
        self.n_phys = sum(npages) + spare
        perm = rng.permutation(self.n_phys)
        self.layout = np.full((len(lengths), self.max_pages), -1, np.int64)
        k = 0
        for s, m in enumerate(npages):
            self.layout[s, :m] = perm[k:k + m]
            k += m
        self.bt = self.layout.astype(np.int32)
        for (s, p), v in (holes or {}).items():
            self.bt[s, p] = v
        self.cache_rows = self.n_phys * page_rows
        self.bt_dev = torch.tensor(self.bt, device=DEV)

    def phys_of(self, s, j):
        """Cache row of entry j of sequence s, or -1 if it is not visible."""
        p = j // self.pr
        if j < 0 or j >= self.lengths[s] or p >= self.max_pages:
            return -1
        pid = int(self.bt[s, p])
        row = pid * self.pr + j % self.pr
        return row if pid >= 0 and row < self.cache_rows else -1

    def visible(self, s):
        n = int(self.lengths[s])
        return np.array([self.phys_of(s, j) >= 0 for j in range(n)], bool)

    def scatter(self, packed, seq_start, junk):
        """Copy each sequence's packed rows to their pages (the layout before
        holes) inside a cache of junk rows."""
        out = junk.clone()
        src, dst = [], []
        for s, n in enumerate(self.lengths):
            j = np.arange(int(n))
            src.append(int(seq_start[s]) + j)
            dst.append(self.layout[s, j // self.pr] * self.pr + j % self.pr)
        src = torch.tensor(np.concatenate(src), device=DEV)
        dst = torch.tensor(np.concatenate(dst), device=DEV)
        out[dst] = packed[src]
        return out


def finite_e4m3_junk(rows, cols, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    b = torch.randint(0, 256, (rows, cols), generator=g, device=DEV, dtype=torch.int32)
    b = torch.where((b & 0x7F) == 0x7F, b - 1, b)            # no NaN patterns
    return b.to(torch.uint8)


def paged_ikeys(wl, pages, seed=1):
    return pages.scatter(wl.ikeys, np_(wl.seq_start), finite_e4m3_junk(pages.cache_rows, wl.cfg.Di, seed))


def expected_selection(scores, visible, K, P):
    """Top-K and pool of one row by brute force: entries ranked by (score
    descending, id ascending), blocks of 8 by (max over visible entries
    descending, id ascending); only visible entries take part; lists ascending
    and -1 padded."""
    ids = np.nonzero(visible)[0]
    sc = scores[ids].astype(np.float64)
    order = np.lexsort((ids, -sc))
    top = np.sort(ids[order[:K]])
    topk = np.full(K, -1, np.int32)
    topk[:len(top)] = top
    pool = None
    if P > 0:
        blocks, first = np.unique(ids // 8, return_index=True)      # ids ascending: blocks are runs
        bmax = np.maximum.reduceat(sc, first) if len(ids) else np.zeros(0)
        border = np.lexsort((blocks, -bmax))
        pb = np.sort(blocks[border[:P]])
        pool = np.full(P, -1, np.int32)
        pool[:len(pb)] = pb
    return topk, pool


def expected_reindex(scores, visible, pool_row, K):
    cand = np.array(sorted(j for b in pool_row if b >= 0 for j in range(8 * b, 8 * b + 8)
                           if j < len(visible) and visible[j]), np.int64)
    sc = scores[cand].astype(np.float64) if len(cand) else np.zeros(0)
    order = np.lexsort((cand, -sc)) if len(cand) else np.zeros(0, np.int64)
    top = np.sort(cand[order[:K]])
    out = np.full(K, -1, np.int32)
    out[:len(top)] = top
    return out


def expected_rows(pages, topk, row_seq):
    """Cache rows of the index lists of rows of sequences row_seq."""
    return np.array([[pages.phys_of(int(row_seq[r]), int(j)) for j in topk[r]] for r in range(topk.shape[0])],
                    np.int32)


def run_full_paged(wl, pages, ikeys, layer, K, P):
    topk, pool, rows = csa2.csa2_index_full_paged(wl.qI[layer], wl.w[layer], ikeys, pages.bt_dev, pages.pr,
                                                  wl.row_seq, wl.row_len, int(max(wl.lengths.max(), 1)), K, P,
                                                  want_pool=P > 0, want_rows=True)
    torch.cuda.synchronize()
    topk = np_(topk)
    assert np.array_equal(np_(rows), expected_rows(pages, topk, np_(wl.row_seq))), "Full: cache rows differ"
    return topk, (np_(pool) if pool is not None else None)


def run_reindex_paged(wl, pages, ikeys, layer, pool, K):
    got, rows = csa2.csa2_index_reindex_paged(wl.qI[layer], wl.w[layer], ikeys, pages.bt_dev, pages.pr, wl.row_seq,
                                              wl.row_len, torch.tensor(pool, device=DEV), K, want_rows=True)
    torch.cuda.synchronize()
    got = np_(got)
    assert np.array_equal(np_(rows), expected_rows(pages, got, np_(wl.row_seq))), "Reindex: cache rows differ"
    return got


FULL_CASES = [
    # name, lengths, page_rows, K, P, idx
    ("ragged_p64", [1, 7, 100, 1000, 4097, 20001], 64, 512, 2048, "int3"),
    ("k_above_p_ties_p32", [40000, 3000, 90], 32, 700, 64, "ties"),
    ("ties_p16", [30000, 17, 8191], 16, 512, 2048, "ties"),
    ("p_below_k_p256", [5000, 3333], 256, 100, 10, "int3"),
    ("long_prefilter_p1024", [150000, 9000], 1024, 1500, 700, "int3"),
    ("empty_row_p8", [0, 900], 8, 32, 40, "int3"),
]


@pytest.mark.parametrize("name,lengths,pr,K,P,idx", FULL_CASES)
def test_index_paged_matches_oracle(name, lengths, pr, K, P, idx):
    log(f"index paged parity: {name}")
    wl = small_workload(lengths, idx_dist=idx)
    pages = Pages(lengths, pr, seed=len(name))
    ikeys = paged_ikeys(wl, pages)
    rows = list(range(len(lengths)))
    topk, pool = run_full_paged(wl, pages, ikeys, 0, K, P)
    rt, rp, packed = oracle_index_rows(wl, 0, rows, K, P)
    assert np.array_equal(topk, rt), f"{name}: top-k differs"
    assert np.array_equal(pool, rp), f"{name}: pool differs"
    want = oracle_reindex_rows(wl, 1, rows, packed, rp, K)
    got = run_reindex_paged(wl, pages, ikeys, 1, rp, K)
    assert np.array_equal(got, want), f"{name}: reindex differs"


def test_index_paged_many_rows_one_sequence():
    """Prefill-like rows (one sequence, causal lengths) over a paged cache
    with an unmapped page."""
    n_seq = 9000
    R = 520
    wl = small_workload([n_seq])
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    wl.row_seq = torch.zeros(R, dtype=torch.int32, device=DEV)
    wl.row_len = torch.arange(n_seq - R + 1, n_seq + 1, dtype=torch.int32, device=DEV)
    wl.qI[0] = workloads.to_e4m3_bytes(torch.randint(-3, 4, (R, 16, 64), generator=g, device=DEV).float())
    wl.w[0] = torch.round(torch.rand(R, 16, generator=g, device=DEV) * 16.0) / 16.0
    pages = Pages([n_seq], 64, seed=4, holes={(0, 7): -1})
    ikeys = paged_ikeys(wl, pages)
    K, P = 64, 100
    topk, pool = run_full_paged(wl, pages, ikeys, 0, K, P)
    scores = oracle.index_scores(np_(wl.qI[0]), np_(wl.w[0]), np_(wl.ikeys), np_(wl.seq_start), np_(wl.row_seq),
                                 np_(wl.row_len), n_seq)
    vis = pages.visible(0)
    for r in [0, 1, 2, 3, 4, 257, R - 2, R - 1]:
        n = int(np_(wl.row_len)[r])
        et, ep = expected_selection(scores[r, :n], vis[:n], K, P)
        assert np.array_equal(topk[r], et) and np.array_equal(pool[r], ep), f"row {r} differs"


def test_index_paged_gemm_path_one_sequence():
    """From 1,024 rows the paged Full call takes the prefill path too (block
    maxima by the GEMM kernel, staged keys read through the block table),
    over a cache with an unmapped page."""
    n_seq = 12000
    R = 1100
    wl = small_workload([n_seq])
    g = torch.Generator(device=DEV)
    g.manual_seed(19)
    wl.row_seq = torch.zeros(R, dtype=torch.int32, device=DEV)
    wl.row_len = torch.arange(n_seq - R + 1, n_seq + 1, dtype=torch.int32, device=DEV)
    wl.qI[0] = workloads.to_e4m3_bytes(torch.randint(-3, 4, (R, 16, 64), generator=g, device=DEV).float())
    wl.w[0] = torch.round(torch.rand(R, 16, generator=g, device=DEV) * 16.0) / 16.0
    pages = Pages([n_seq], 64, seed=5, holes={(0, 11): -1, (0, 150): 10 ** 6})
    ikeys = paged_ikeys(wl, pages)
    K, P = 64, 100
    topk, pool = run_full_paged(wl, pages, ikeys, 0, K, P)
    scores = oracle.index_scores(np_(wl.qI[0]), np_(wl.w[0]), np_(wl.ikeys), np_(wl.seq_start), np_(wl.row_seq),
                                 np_(wl.row_len), n_seq)
    vis = pages.visible(0)
    for r in [0, 1, 7, 8, 9, 513, R - 9, R - 8, R - 1]:
        n = int(np_(wl.row_len)[r])
        et, ep = expected_selection(scores[r, :n], vis[:n], K, P)
        assert np.array_equal(topk[r], et) and np.array_equal(pool[r], ep), f"row {r} differs"


def test_index_paged_unmapped_pages():
    lengths = [20000, 3001, 640]
    pr = 64
    holes = {(0, 3): -1, (0, 100): -1, (0, 312): 10 ** 6,     # two holes and a page past the cache
             (1, 46): -1,                                      # the ragged last page
             (2, 0): -1, (2, 1): -1, (2, 2): -1, (2, 3): -1, (2, 4): -1, (2, 5): -1, (2, 6): -1,
             (2, 7): -1, (2, 8): -1, (2, 9): -1}               # every page: nothing visible
    pages = Pages(lengths, pr, seed=5, holes=holes)
    wl = small_workload(lengths)
    ikeys = paged_ikeys(wl, pages)
    R = len(lengths)
    K, P = 300, 500
    topk, pool = run_full_paged(wl, pages, ikeys, 0, K, P)
    scores = {}
    for layer in (0, 1):
        scores[layer] = oracle.index_scores(np_(wl.qI[layer]), np_(wl.w[layer]), np_(wl.ikeys),
                                            np_(wl.seq_start), np_(wl.row_seq), np_(wl.row_len), max(lengths))
    for r in range(R):
        vis = pages.visible(r)
        et, ep = expected_selection(scores[0][r, :lengths[r]], vis, K, P)
        assert np.array_equal(topk[r], et), f"row {r}: top-k differs"
        assert np.array_equal(pool[r], ep), f"row {r}: pool differs"
    assert (topk[2] == -1).all() and (pool[2] == -1).all()
    got = run_reindex_paged(wl, pages, ikeys, 1, pool, K)
    for r in range(R):
        er = expected_reindex(scores[1][r, :lengths[r]], pages.visible(r), pool[r], K)
        assert np.array_equal(got[r], er), f"row {r}: reindex differs"


def test_index_reindex_paged_unsorted_pool():
    """An out-of-order pool with -1 and out-of-range ids (sorted in the
    selector) over a paged cache: the oracle's Top-K and the matching rows."""
    lengths = [3000, 700]
    wl = small_workload(lengths)
    pages = Pages(lengths, 16, seed=12)
    ikeys = paged_ikeys(wl, pages)
    rng = np.random.default_rng(6)
    K, P = 60, 48
    pool = np.full((2, P), -1, np.int32)
    for r, n in enumerate(lengths):
        nb = (n + 7) // 8
        ids = rng.choice(nb, 40, replace=False)
        ids[5] = nb + 9                                  # out of range: skipped
        pool[r, rng.permutation(P)[:40]] = ids
    packed = oracle_index_rows(wl, 0, [0, 1], K, P)[2]
    want = oracle_reindex_rows(wl, 1, [0, 1], packed, pool, K)
    got = run_reindex_paged(wl, pages, ikeys, 1, pool, K)
    assert np.array_equal(got, want)


def test_paged_rows_formula():
    lengths = [9000, 700, 30000]
    pages = Pages(lengths, 128, seed=3, holes={(0, 10): -1, (2, 200): 1 << 20})
    R, K = len(lengths), 700
    rng = np.random.default_rng(4)
    idx = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        idx[r, :k] = rng.permutation(n)[:k]
        idx[r, 5] = n                        # past the row: -1
        idx[r, 6] = -7
    idx[0, 7] = 10 * 128 + 3                 # inside the hole
    row_seq = torch.arange(R, dtype=torch.int32, device=DEV)
    row_len = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    got = np_(csa2.csa2_paged_rows(pages.bt_dev, pages.pr, pages.cache_rows, row_seq, row_len,
                                   torch.tensor(idx, device=DEV)))
    want = np.array([[pages.phys_of(r, int(j)) for j in idx[r]] for r in range(R)], np.int32)
    assert np.array_equal(got, want)
    assert got[0, 7] == -1 and (got[:, 5] == -1).all()


def paged_kv(wl, pages, seed=2):
    """The packed FP4 cache and a paged copy of it (junk in unused rows)."""
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), codes, scales)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    junk_codes = torch.randint(0, 256, (pages.cache_rows, D // 2), generator=g, device=DEV,
                               dtype=torch.int32).to(torch.uint8)
    pc = pages.scatter(codes, np_(wl.seq_start), junk_codes)
    ps = pages.scatter(scales, np_(wl.seq_start), finite_e4m3_junk(pages.cache_rows, D // 16, seed + 1))
    return codes, scales, pc, ps


def ring_copy(wl, layer, heads, W, seed=3):
    """SWA rows of each row r stored as a ring: window row i in slot
    (heads[r] + i) mod W of the row's W slots; other rows junk."""
    swa = wl.swa[layer]
    ring = finite_e4m3_junk(swa.shape[0], swa.shape[1], seed)
    starts = np_(wl.swa_row_start)
    for r, h in enumerate(heads):
        i = np.arange(W)
        src = torch.tensor(int(starts[r]) + i, device=DEV)
        dst = torch.tensor(int(starts[r]) + (int(h) + i) % W, device=DEV)
        ring[dst] = swa[src]
    return ring


ATTN_CASES = [
    # name, lengths, D, H, K, W, page_rows
    ("d512_h64_split_p64", [9000, 700, 30000], 512, 64, 512, 128, 64),
    ("d512_h64_many_rows_nosplit_p16", [300 + 37 * i for i in range(130)], 512, 64, 512, 128, 16),
    ("d256_h24_k100_w7_p8", [1000, 77, 5000, 2222], 256, 24, 100, 7, 8),
    ("d128_h8_k64_w32_p256", [4096, 5000], 128, 8, 64, 32, 256),
]


@pytest.mark.parametrize("name,lengths,D,H,K,W,pr", ATTN_CASES)
def test_sparse_attn_phys_matches_packed_and_oracle(name, lengths, D, H, K, W, pr):
    log(f"sparse_attn_phys parity: {name}")
    R = len(lengths)
    wl = small_workload(lengths, D=D, H=H, W=W, Hi=8, Di=64)
    holes = {(0, 2): -1, (R - 1, 1): -1}
    pages = Pages(lengths, pr, seed=len(name), holes=holes)
    codes, scales, pc, ps = paged_kv(wl, pages)
    rng = np.random.default_rng(len(name) + 1)
    topk = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        topk[r, :k] = np.sort(rng.choice(n, k, replace=False))
        if k >= 4:
            topk[r, 1] = -1
            topk[r, 2] = n + 3
    if W > 0:
        sl = np_(wl.swa_len)
        sl[0] = W // 2
        if R > 2:
            sl[1] = 0
        wl.swa_len = torch.tensor(sl, device=DEV)
    heads = rng.integers(0, W, R).astype(np.int32)
    heads[0] = W - 1                         # the window wraps right away
    if R > 2:
        heads[2] = -3                        # taken mod W
    if R > 3:
        heads[3] = W + 2
    scale = 1.0 / math.sqrt(D)
    topk_t = torch.tensor(topk, device=DEV)
    phys = csa2.csa2_paged_rows(pages.bt_dev, pr, pages.cache_rows, wl.row_seq, wl.row_len, topk_t)
    # the packed call sees the same key set: hole entries removed from the lists
    vis = np.array([[pages.phys_of(r, int(j)) >= 0 for j in topk[r]] for r in range(R)])
    masked = np.where(vis, topk, -1).astype(np.int32)
    out_p, lse_p = csa2.csa2_sparse_attn(wl.q[0], codes, scales, wl.seq_start, wl.row_seq, wl.row_len,
                                         torch.tensor(masked, device=DEV), wl.swa[0], wl.swa_row_start,
                                         wl.swa_len, W, scale)
    out_f, lse_f = csa2.csa2_sparse_attn_phys(wl.q[0], pc, ps, phys, wl.swa[0], wl.swa_row_start, wl.swa_len, W,
                                              scale)
    ring = ring_copy(wl, 0, heads, W)
    out_r, lse_r = csa2.csa2_sparse_attn_phys(wl.q[0], pc, ps, phys, ring, wl.swa_row_start, wl.swa_len, W, scale,
                                              swa_head=torch.tensor(heads, device=DEV))
    torch.cuda.synchronize()
    out_p, lse_p = np_(out_p), np_(lse_p)
    assert np.array_equal(np_(out_f), out_p) and np.array_equal(np_(lse_f), lse_p), f"{name}: phys != packed"
    assert np.array_equal(np_(out_r), out_p) and np.array_equal(np_(lse_r), lse_p), f"{name}: ring != packed"
    check_rows = list(range(R)) if R <= 8 else [0, 1, 2, R // 2, R - 1]
    ref = oracle_attn_rows(wl, {r: masked[r] for r in check_rows}, 0, check_rows, W, scale)
    check_attn(np_(out_r)[check_rows], np.stack([ref[r][0] for r in check_rows]), np_(lse_r)[check_rows],
               np.stack([ref[r][1] for r in check_rows]), what=name)


def test_sparse_attn_phys_cache_beyond_2gib():
    """Cache rows past 2^31 bytes of codes (9.4M rows at D = 512): the row form
    reads them through 64-bit addresses, matches the packed call and meets the
    oracle's outputs."""
    lengths = [3000, 5000]
    D, H, K, W, pr = 512, 16, 128, 32, 64
    wl = small_workload(lengths, D=D, H=H, W=W, Hi=8, Di=64)
    pages = Pages(lengths, pr, seed=2)
    off_pages = (9_400_000 + pr - 1) // pr                 # every page beyond 2^31 bytes of codes
    rows_total = (off_pages + pages.n_phys) * pr
    codes, scales, pc, ps = paged_kv(wl, pages)
    big_c = torch.empty(rows_total, D // 2, dtype=torch.uint8, device=DEV)
    big_s = torch.empty(rows_total, D // 16, dtype=torch.uint8, device=DEV)
    big_c[off_pages * pr:] = pc
    big_s[off_pages * pr:] = ps
    bt = torch.where(pages.bt_dev >= 0, pages.bt_dev + off_pages, pages.bt_dev)
    rng = np.random.default_rng(3)
    topk = np.full((2, K), -1, np.int32)
    for r, n in enumerate(lengths):
        topk[r] = np.sort(rng.choice(n, K, replace=False))
    topk_t = torch.tensor(topk, device=DEV)
    phys = csa2.csa2_paged_rows(bt, pr, rows_total, wl.row_seq, wl.row_len, topk_t)
    assert int(phys.min()) >= off_pages * pr
    scale = 1.0 / math.sqrt(D)
    out_p, lse_p = csa2.csa2_sparse_attn(wl.q[0], codes, scales, wl.seq_start, wl.row_seq, wl.row_len, topk_t,
                                         wl.swa[0], wl.swa_row_start, wl.swa_len, W, scale)
    out_f, lse_f = csa2.csa2_sparse_attn_phys(wl.q[0], big_c, big_s, phys, wl.swa[0], wl.swa_row_start, wl.swa_len,
                                              W, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_p) and torch.equal(lse_f, lse_p)
    ref = oracle_attn_rows(wl, {r: topk[r] for r in range(2)}, 0, [0, 1], W, scale)
    check_attn(np_(out_f), np.stack([ref[r][0] for r in range(2)]), np_(lse_f),
               np.stack([ref[r][1] for r in range(2)]), what="rows beyond 2 GiB")


@pytest.mark.parametrize("cid", [1, 2])
def test_paged_step_matches_packed_step(cid):
    """The whole layer schedule over a paged cache (shuffled pages of 64
    entries, SWA windows as rings) gives the packed schedule's indices and
    outputs bit for bit, and the paged step's own outputs match the oracle,
    whose layer schedule decides which Top-K list each layer attends with."""
    from sparse_attention_fp4_amd.step import CSA2Step
    log(f"paged step vs packed step: config {cid}")
    cfg = workloads.CONFIGS[cid]
    wl = workloads.make(cfg, DEV)
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), codes, scales)
    new_kv = wl.kv_raw[wl.new_rows].contiguous()
    common = dict(row_seq=wl.row_seq, row_len=wl.row_len, max_len=int(wl.lengths.max()), new_kv=new_kv, qI=wl.qI,
                  w=wl.w, q=wl.q, swa_row_start=wl.swa_row_start, swa_len=wl.swa_len, W=cfg.W, K=cfg.K, P=cfg.P,
                  softmax_scale=1.0 / math.sqrt(D))
    lay = workloads.paged_layout(wl.lengths, 64, seed=cid, device=DEV, spare_pages=5)
    pc, ps, pk = (workloads.to_pages(lay, t) for t in (codes, scales, wl.ikeys))
    g = torch.Generator(device=DEV)
    g.manual_seed(cid)
    head = torch.randint(0, cfg.W, (wl.R,), generator=g, device=DEV, dtype=torch.int32)
    ring = {l: workloads.swa_ring(t, wl.swa_row_start, cfg.W, head) for l, t in wl.swa.items()}
    packed = CSA2Step(list(cfg.layers), codes=codes, scales=scales, ikeys=wl.ikeys, seq_start=wl.seq_start,
                      new_rows=wl.new_rows, swa=wl.swa, **common)
    paged = CSA2Step(list(cfg.layers), codes=pc, scales=ps, ikeys=pk, seq_start=None, new_rows=lay.dst[wl.new_rows],
                     swa=ring, block_table=lay.block_table, page_rows=64, swa_head=head, **common)
    packed.run()
    paged.run()
    torch.cuda.synchronize()
    assert torch.equal(pc[lay.dst], codes) and torch.equal(ps[lay.dst], scales)
    for l in packed.topk:
        assert torch.equal(packed.topk[l], paged.topk[l]), f"layer {l}: indices differ"
    assert torch.equal(packed.pool, paged.pool)
    for l in range(len(cfg.layers)):
        assert torch.equal(packed.out[l], paged.out[l]), f"layer {l}: output differs"
        assert torch.equal(packed.lse[l], paged.lse[l]), f"layer {l}: lse differs"
    # the paged step against the oracle directly
    modes = list(cfg.layers)
    rows_chk = list(range(wl.R)) if wl.R <= 4 else [0, wl.R // 2, wl.R - 1]
    rt, rp, packed_o = oracle_index_rows(wl, 0, rows_chk, cfg.K, cfg.P)
    assert np.array_equal(np_(paged.topk[0])[rows_chk], rt), "paged Full top-k != oracle"
    assert np.array_equal(np_(paged.pool)[rows_chk], rp), "paged pool != oracle"
    otk = {0: rt}
    for l, m in enumerate(modes):
        if m == "R":
            otk[l] = oracle_reindex_rows(wl, l, rows_chk, packed_o, rp, cfg.K)
            assert np.array_equal(np_(paged.topk[l])[rows_chk], otk[l]), f"paged Reindex layer {l} != oracle"
    par = oracle.step.parents(modes)
    for l in sorted({0, modes.index("R"), len(modes) - 1}):
        ref = oracle_attn_rows(wl, {r: otk[par[l]][i] for i, r in enumerate(rows_chk)}, l, rows_chk, cfg.W,
                               1.0 / math.sqrt(D))
        check_attn(np_(paged.out[l])[rows_chk], np.stack([ref[r][0] for r in rows_chk]),
                   np_(paged.lse[l])[rows_chk], np.stack([ref[r][1] for r in rows_chk]),
                   what=f"paged step config {cid} layer {l}")
