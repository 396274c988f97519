"""csa2_index_reindex_noalloc (the Reindex call whose score buffer is the
library's fixed device array, for callers that cannot allocate) through the C
ABI, against csa2_index_reindex with a caller workspace: bit-identical Top-K
lists on two calls in a row, the second with fewer rows, shorter rows and a
different query, so a result left in the array by the first call cannot pass
for the second.  Also the size limit: too many rows are refused."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_attention_fp4_amd as csa2

pytestmark = pytest.mark.gpu
DEV = "cuda"


def p(t):
    return ctypes.c_void_p(t.data_ptr())


def case(R, n, seed, Hi=64, Di=128, K=512, P=2048):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    e4m3 = lambda *s: torch.randint(-3, 4, s, generator=g, device=DEV).float().to(torch.float8_e4m3fn).view(
        torch.uint8)
    lens = torch.randint(n // 2, n + 1, (R,), generator=g, device=DEV, dtype=torch.int32)
    starts = torch.zeros(R, dtype=torch.int64, device=DEV)
    starts[1:] = torch.cumsum(lens.long(), 0)[:-1]
    keys = e4m3(int(lens.sum()), Di)
    qF, qR = e4m3(R, Hi, Di), e4m3(R, Hi, Di)
    w = torch.round(torch.rand(R, Hi, generator=g, device=DEV) * 16) / 16
    rs = torch.arange(R, dtype=torch.int32, device=DEV)
    _, pool = csa2.csa2_index_full(qF, w, keys, starts, rs, lens, int(lens.max()), K, P)
    return dict(qI=qR, w=w, keys=keys, starts=starts, rs=rs, lens=lens, pool=pool, R=R, Hi=Hi, Di=Di, K=K, P=P)


def with_workspace(c):
    return csa2.csa2_index_reindex(c["qI"], c["w"], c["keys"], c["starts"], c["rs"], c["lens"], c["pool"], c["K"])


def noalloc(c):
    L = csa2.lib()
    out = torch.full((c["R"], c["K"]), -7, dtype=torch.int32, device=DEV)
    st = L.csa2_index_reindex_noalloc(p(c["qI"]), p(c["w"]), p(c["keys"]), p(c["starts"]), p(c["rs"]), p(c["lens"]),
                                      p(c["pool"]), c["R"], c["Hi"], c["Di"], c["K"], c["P"], 8, p(out),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.csa2_last_error()
    return out


def test_noalloc_reindex_matches_workspace_form_on_two_calls():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    first = case(R=200, n=40000, seed=1)
    second = case(R=7, n=9000, seed=2)
    for c in (first, second):
        got = noalloc(c)
        torch.cuda.synchronize()
        want = with_workspace(c)
        torch.cuda.synchronize()
        assert torch.equal(got, want)
        assert int((got >= 0).sum()) == c["R"] * c["K"]      # every row has at least K candidates
    # the Python binding of the same entry point
    out = torch.empty(second["R"], second["K"], dtype=torch.int32, device=DEV)
    csa2.csa2_index_reindex_noalloc(second["qI"], second["w"], second["keys"], second["starts"], second["rs"],
                                    second["lens"], second["pool"], second["K"], out)
    torch.cuda.synchronize()
    assert torch.equal(out, with_workspace(second))


def test_noalloc_reindex_refuses_more_rows_than_the_array_holds():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L = csa2.lib()
    fake = ctypes.c_void_p(0x1000)
    # 257 rows x 2048 pool blocks x 8 positions x 4 B > 16 MiB: refused before any HIP call
    st = L.csa2_index_reindex_noalloc(fake, fake, fake, fake, fake, fake, fake, 257, 64, 128, 512, 2048, 8, fake,
                                      None)
    assert st == 3 and b"scratch" in L.csa2_last_error()
