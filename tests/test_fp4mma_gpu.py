"""GPU checks of csa2_sparse_attn_fp4mma, the form of the attention call whose
query-key products for the selected FP4 entries run on the scaled FP4
matrix-core product (codes straight from the cache) wherever that product is
exact.

The FP4 KV cache (section 一 of the teardown "DeepSeek V4.1 Flash 拆解",
FP4 KV cache paragraph) keeps one E4M3 scale per 16 channels; the hardware
product takes one power-of-two scale per 32 channels.  So:

* on caches whose two E4M3 scales of every 32-channel block are the same
  power of two, with queries exact as E4M3 under one power-of-two scale per
  32 channels and values on a grid whose fp32 sums are exact, every Top-K
  fragment takes the native product and the outputs equal those of
  csa2_sparse_attn bit for bit (and the oracle within the attention
  tolerance);
* on ordinary caches (scales with mantissa bits) or queries that are not
  exact in E4M3, no fragment takes it and the outputs again equal
  csa2_sparse_attn bit for bit;
* on a mix, exactly the fragments whose entries all qualify take it.

The inputs are seeded and synthetic; the cache bytes are drawn directly
(codes uniform over all 16 E2M1 codes), and the oracle reads the same bytes.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_fp4_amd as csa2
import workloads
from helpers import bits16, check_attn, log, np_

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


def p2_scales(rng, rows, D, lo=-2, hi=2):
    """E4M3 scale bytes: one power of two 2^k (k in [lo, hi]) per 32-channel
    block, the same byte for both 16-channel groups of the block."""
    k = rng.integers(lo, hi + 1, size=(rows, D // 32))
    b = ((k + 7) << 3).astype(np.uint8)   # E4M3 2^(e - 7): exponent field e = k + 7, mantissa 0
    return np.repeat(b, 2, axis=1)


def grid_query(rng, R, H, D):
    """bf16 queries on the grid 2^-3 * {-15 .. 15}: exact as E4M3 under one
    power-of-two scale per 32 channels (4 significant bits)."""
    v = rng.integers(-15, 16, size=(R, H, D)).astype(np.float32) / 8.0
    return torch.tensor(v, device=DEV).to(torch.bfloat16)


def make_case(seed, lengths, D, H, K, W, scales="p2", query="grid"):
    rng = np.random.default_rng(seed)
    R = len(lengths)
    rows = int(sum(lengths))
    codes = rng.integers(0, 256, size=(rows, D // 2), dtype=np.uint8)
    if scales == "p2":
        sc = p2_scales(rng, rows, D)
    elif scales == "ordinary":
        # E4M3 scales with mantissa bits: 1.125 .. 1.875 x 2^k
        sc = ((rng.integers(5, 9, size=(rows, D // 16)) << 3) | rng.integers(1, 8, size=(rows, D // 16))).astype(
            np.uint8)
    else:   # mixed: the entries of odd sequences get a mantissa bit in their first group's scale
        sc = p2_scales(rng, rows, D)
        starts = np.concatenate([[0], np.cumsum(lengths)])
        for b in range(1, len(lengths), 2):
            sc[starts[b]:starts[b + 1], 0] |= 1
    seq_start = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    row_seq = np.arange(R, dtype=np.int32)
    row_len = np.array(lengths, np.int32)
    topk = np.full((R, K), -1, np.int32)
    for r, n in enumerate(lengths):
        k = min(K, n)
        topk[r, :k] = np.sort(rng.choice(n, k, replace=False))
        if k >= 4:
            topk[r, 1] = -1        # a hole
    # SWA rows: E4M3 bytes of small integers (both forms dequantise them alike)
    swa_vals = rng.integers(-6, 7, size=(R * max(W, 1), D)).astype(np.float32)
    swa = torch.tensor(swa_vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    swa_row_start = (np.arange(R) * max(W, 1)).astype(np.int64)
    swa_len = np.full(R, W, np.int32)
    if query == "grid":
        q = grid_query(rng, R, H, D)
    else:
        q = torch.tensor(rng.standard_normal((R, H, D)).astype(np.float32), device=DEV).to(torch.bfloat16)
    t = lambda a: torch.tensor(a, device=DEV)
    return dict(q=q, codes=t(codes), scales=t(sc), seq_start=t(seq_start), row_seq=t(row_seq), row_len=t(row_len),
                topk=t(topk), swa=t(swa), swa_row_start=t(swa_row_start), swa_len=t(swa_len), W=W,
                scale=1.0 / math.sqrt(D))


def run(c, fp4mma):
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    args = (c["q"], c["codes"], c["scales"], c["seq_start"], c["row_seq"], c["row_len"], c["topk"], c["swa"],
            c["swa_row_start"], c["swa_len"], c["W"], c["scale"])
    if fp4mma:
        out, lse = csa2.csa2_sparse_attn_fp4mma(*args, native_fragments=cnt)
    else:
        out, lse = csa2.csa2_sparse_attn(*args)
    torch.cuda.synchronize()
    return out, lse, int(cnt.item())


def oracle_rows(c, rows):
    out, lse = oracle.sparse_attn(bits16(c["q"])[rows], np_(c["codes"]), np_(c["scales"]), np_(c["seq_start"]),
                                  np_(c["row_seq"])[rows], np_(c["row_len"])[rows], np_(c["topk"])[rows],
                                  np_(c["swa"]), np_(c["swa_row_start"])[rows], np_(c["swa_len"])[rows], c["W"],
                                  c["scale"])
    return out, lse


def topk_fragments(R, H, D, K, W):
    """Top-K fragments the kernels score: per (row, head group), ceil(K/16)."""
    heads16 = (H + 15) // 16
    ht = min(512 // D, heads16)
    ht = 2 if ht == 3 else ht
    hg = (H + 16 * ht - 1) // (16 * ht)
    if R * hg < 256:
        hg = heads16
    return R * hg * ((K + 15) // 16)


CASES = [
    ("d512_h64_rows24_two_splits", [3000 + 97 * i for i in range(24)], 512, 64, 512, 128),
    ("d512_h16_rows3_many_splits", [9000, 2000, 600], 512, 16, 512, 128),
    ("d128_h8_rows5", [4096, 300, 1000, 77, 2500], 128, 8, 64, 32),
    ("d256_h32_rows4", [5000, 301, 900, 64], 256, 32, 100, 16),
]


@pytest.mark.parametrize("name,lengths,D,H,K,W", CASES)
def test_fp4mma_equals_dequant_path_on_exact_subset(name, lengths, D, H, K, W):
    log(f"fp4mma exact subset: {name}")
    c = make_case(11 + len(name), lengths, D, H, K, W)
    R = len(lengths)
    o0, l0, _ = run(c, False)
    o1, l1, n = run(c, True)
    assert n == topk_fragments(R, H, D, K, W), n
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    rows = [0, R // 2, R - 1]
    ro, rl = oracle_rows(c, rows)
    check_attn(np_(o1)[rows], ro, np_(l1)[rows], rl, what=f"fp4mma {name}")


@pytest.mark.parametrize("scales,query", [("ordinary", "grid"), ("p2", "normal")])
def test_fp4mma_falls_back_where_not_exact(scales, query):
    """Scales with mantissa bits, or a query not exact in E4M3: no fragment
    takes the native product, and the call is csa2_sparse_attn bit for bit."""
    lengths, D, H, K, W = [4000, 900, 2500], 512, 64, 512, 128
    c = make_case(5, lengths, D, H, K, W, scales=scales, query=query)
    o0, l0, _ = run(c, False)
    o1, l1, n = run(c, True)
    assert n == 0
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_fp4mma_mixed_cache():
    """Rows of even sequences qualify, rows of odd ones do not: exactly the
    former's fragments take the native product, and every row equals
    csa2_sparse_attn bit for bit and the oracle within tolerance."""
    lengths, D, H, K, W = [6000, 3000, 2000, 4000], 512, 64, 64, 128
    c = make_case(9, lengths, D, H, K, W, scales="mixed")
    o0, l0, _ = run(c, False)
    o1, l1, n = run(c, True)
    assert n == topk_fragments(len(lengths), H, D, K, W) // 2, n
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    ro, rl = oracle_rows(c, [0, 1, 2, 3])
    check_attn(np_(o1), ro, np_(l1), rl, what="fp4mma mixed")


def test_fp4mma_quantised_cache_matches_oracle():
    """An ordinary quantised cache (csa2_quantize_append of N(0,1) values)
    through the native-FP4 form: the oracle's tolerance, like csa2_sparse_attn."""
    cfg = workloads.Config(97, "small", B=3, N=None, D=512, W=64, H=64, Hi=8, Di=64, K=0, P=0, idx_dist="int3",
                           w_dist="u01_16", layers="F", kv_dist="normal")
    wl = workloads.make(cfg, DEV, lengths=np.array([3000, 800, 5000]))
    rows, D = wl.kv_raw.shape
    codes = torch.empty(rows, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(rows, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(wl.kv_raw, torch.arange(rows, dtype=torch.int64, device=DEV), codes, scales)
    rng = np.random.default_rng(4)
    K = 256
    topk = np.full((3, K), -1, np.int32)
    for r, n in enumerate([3000, 800, 5000]):
        topk[r] = np.sort(rng.choice(n, K, replace=False))
    c = dict(q=wl.q[0], codes=codes, scales=scales, seq_start=wl.seq_start, row_seq=wl.row_seq, row_len=wl.row_len,
             topk=torch.tensor(topk, device=DEV), swa=wl.swa[0], swa_row_start=wl.swa_row_start,
             swa_len=wl.swa_len, W=64, scale=1.0 / math.sqrt(D))
    o0, l0, _ = run(c, False)
    o1, l1, n = run(c, True)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    ro, rl = oracle_rows(c, [0, 1, 2])
    check_attn(np_(o1), ro, np_(l1), rl, what="fp4mma quantised cache")
