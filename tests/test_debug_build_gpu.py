"""The debug build (libcsa2_debug.so, compiled with -DCSA2_DEBUG) through the
C ABI: calls whose device-side inputs hold out-of-range values (an index past
its row, a pool block past the row, a duplicated pool block, a row length past
max_len, a window length past W, a destination row past the cache) return
CSA2_ERR_DEVICE_CHECK, found by the kernels' own range checks, and otherwise
return CSA2_OK with the release build's outputs, bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as csa2
from sparse_attention_fp4_amd.build import LIB_DEBUG

pytestmark = pytest.mark.gpu
DEV = "cuda"
OK, DEVICE_CHECK = 0, 6


@pytest.fixture(scope="module")
def dbg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    return csa2.load(LIB_DEBUG)


def p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def small_index(n=3000, R=2, Hi=16, Di=64, seed=0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    keys = torch.randint(-3, 4, (n, Di), generator=g, device=DEV).float().to(torch.float8_e4m3fn).view(torch.uint8)
    qI = torch.randint(-3, 4, (R, Hi, Di), generator=g, device=DEV).float().to(torch.float8_e4m3fn).view(torch.uint8)
    w = torch.ones(R, Hi, device=DEV)
    return keys, qI, w


def call_full(L, qI, w, keys, row_len, max_len, K, P):
    R, Hi, Di = qI.shape
    topk = torch.empty(R, K, dtype=torch.int32, device=DEV)
    pool = torch.empty(R, P, dtype=torch.int32, device=DEV)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    rs = torch.zeros(R, dtype=torch.int32, device=DEV)
    nb = L.csa2_index_full_workspace_bytes(R, max_len, Hi, K, P, 8)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    st = L.csa2_index_full(p(qI), p(w), p(keys), p(ss), p(rs), p(row_len), R, Hi, Di, max_len, K, P, 8, p(topk),
                           p(pool), p(ws), ws.numel(), stream())
    torch.cuda.synchronize()
    return st, topk, pool


def test_index_full_row_len_past_max_len(dbg):
    keys, qI, w = small_index()
    good = torch.tensor([2000, 2500], dtype=torch.int32, device=DEV)
    st_d, t_d, p_d = call_full(dbg, qI, w, keys, good, 2500, 64, 32)
    st_r, t_r, p_r = call_full(csa2.lib(), qI, w, keys, good, 2500, 64, 32)
    assert st_d == OK and st_r == OK
    assert torch.equal(t_d, t_r) and torch.equal(p_d, p_r)
    bad = torch.tensor([2000, 2900], dtype=torch.int32, device=DEV)   # past max_len = 2500
    st_d, _, _ = call_full(dbg, qI, w, keys, bad, 2500, 64, 32)
    assert st_d == DEVICE_CHECK, dbg.csa2_last_error()
    assert b"out-of-range" in dbg.csa2_last_error()
    # the count was cleared: a good call afterwards is OK again
    st_d, t_d2, _ = call_full(dbg, qI, w, keys, good, 2500, 64, 32)
    assert st_d == OK and torch.equal(t_d2, t_r)


def call_reindex(L, qI, w, keys, row_len, pool, K):
    R, Hi, Di = qI.shape
    P = pool.shape[1]
    topk = torch.empty(R, K, dtype=torch.int32, device=DEV)
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    rs = torch.zeros(R, dtype=torch.int32, device=DEV)
    nb = L.csa2_index_reindex_workspace_bytes(R, Hi, K, P, 8)
    ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=DEV)
    st = L.csa2_index_reindex(p(qI), p(w), p(keys), p(ss), p(rs), p(row_len), p(pool), R, Hi, Di, K, P, 8, p(topk),
                              p(ws), ws.numel(), stream())
    torch.cuda.synchronize()
    return st, topk


def test_index_reindex_bad_and_duplicate_pool_ids(dbg):
    keys, qI, w = small_index()
    row_len = torch.tensor([2000, 2500], dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(1)
    pool_np = np.stack([np.sort(rng.choice(250, 32, replace=False)) for _ in range(2)]).astype(np.int32)
    pool = torch.tensor(pool_np, device=DEV)
    st_d, t_d = call_reindex(dbg, qI, w, keys, row_len, pool, 64)
    st_r, t_r = call_reindex(csa2.lib(), qI, w, keys, row_len, pool, 64)
    assert st_d == OK and st_r == OK and torch.equal(t_d, t_r)
    past = pool.clone()
    past[0, 5] = 10_000                      # past the row's 250 blocks
    assert call_reindex(dbg, qI, w, keys, row_len, past, 64)[0] == DEVICE_CHECK
    dup = pool.clone()
    dup[1, 7] = dup[1, 6]                    # listed twice: counts once in release, reported in debug
    st_d, t_dup_d = call_reindex(dbg, qI, w, keys, row_len, dup, 64)
    assert st_d == DEVICE_CHECK
    st_r, t_dup_r = call_reindex(csa2.lib(), qI, w, keys, row_len, dup, 64)
    assert st_r == OK and torch.equal(t_dup_d, t_dup_r)
    # counting the duplicate once equals dropping it
    drop = pool.clone()
    drop[1, 7] = -1
    assert torch.equal(t_dup_r, call_reindex(csa2.lib(), qI, w, keys, row_len, drop, 64)[1])


def call_attn(L, q, codes, scales, row_len, topk, swa, swa_len, W, fp4mma=False):
    R, H, D = q.shape
    K = topk.shape[1]
    ss = torch.zeros(1, dtype=torch.int64, device=DEV)
    rs = torch.zeros(R, dtype=torch.int32, device=DEV)
    srs = torch.zeros(R, dtype=torch.int64, device=DEV)
    out = torch.empty(R, H, D, device=DEV)
    lse = torch.empty(R, H, device=DEV)
    nb = L.csa2_sparse_attn_workspace_bytes(R, H, D, K, W)
    ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=DEV)
    args = [p(q), p(codes), p(scales), p(ss), p(rs), p(row_len), p(topk), K, p(swa), p(srs), p(swa_len), R, H, D, W,
            ctypes.c_float(D ** -0.5), p(out), p(lse)]
    if fp4mma:
        st = L.csa2_sparse_attn_fp4mma(*args, None, p(ws), ws.numel(), stream())
    else:
        st = L.csa2_sparse_attn(*args, p(ws), ws.numel(), stream())
    torch.cuda.synchronize()
    return st, out, lse


# two rows (eight-wave workgroups, split keys); 2,048 rows (four-wave
# workgroups); the native-FP4 form
@pytest.mark.parametrize("R,fp4mma", [(2, False), (2048, False), (2, True)])
def test_sparse_attn_bad_ids_and_window(dbg, R, fp4mma):
    H, D, K, W, n = 16, 128, 64, 16, 1000
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    kv = torch.randn(n, D, generator=g, device=DEV)
    codes = torch.empty(n, D // 2, dtype=torch.uint8, device=DEV)
    scales = torch.empty(n, D // 16, dtype=torch.uint8, device=DEV)
    csa2.csa2_quantize_append(kv, torch.arange(n, dtype=torch.int64, device=DEV), codes, scales)
    q = torch.randn(R, H, D, generator=g, device=DEV).to(torch.bfloat16)
    swa = torch.randn(W, D, generator=g, device=DEV).to(torch.float8_e4m3fn).view(torch.uint8)
    row_len = torch.full((R,), n, dtype=torch.int32, device=DEV)
    topk = torch.stack([torch.randperm(n, generator=g, device=DEV)[:K].sort().values for _ in range(R)]).int()
    topk[:, -4:] = -1
    swa_len = torch.full((R,), W, dtype=torch.int32, device=DEV)
    st_d, o_d, l_d = call_attn(dbg, q, codes, scales, row_len, topk, swa, swa_len, W, fp4mma)
    st_r, o_r, l_r = call_attn(csa2.lib(), q, codes, scales, row_len, topk, swa, swa_len, W, fp4mma)
    assert st_d == OK and st_r == OK
    assert torch.equal(o_d, o_r) and torch.equal(l_d, l_r)
    bad = topk.clone()
    bad[1, 3] = n + 5                        # past the row
    assert call_attn(dbg, q, codes, scales, row_len, bad, swa, swa_len, W, fp4mma)[0] == DEVICE_CHECK
    long_w = swa_len.clone()
    long_w[0] = W + 1                        # window longer than W
    assert call_attn(dbg, q, codes, scales, row_len, topk, swa, long_w, W, fp4mma)[0] == DEVICE_CHECK


def test_quantize_destination_past_cache(dbg):
    x = torch.randn(4, 64, device=DEV)
    codes = torch.zeros(10, 32, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(10, 4, dtype=torch.uint8, device=DEV)
    dst = torch.tensor([0, 3, 12, 9], dtype=torch.int64, device=DEV)
    st = dbg.csa2_quantize_append(p(x), 0, 4, 64, p(dst), p(codes), p(scales), 10, stream())
    torch.cuda.synchronize()
    assert st == DEVICE_CHECK
    ok = torch.tensor([0, 3, 5, 9], dtype=torch.int64, device=DEV)
    st = dbg.csa2_quantize_append(p(x), 0, 4, 64, p(ok), p(codes), p(scales), 10, stream())
    torch.cuda.synchronize()
    assert st == OK
