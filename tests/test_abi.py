"""The C ABI on a host without a GPU: the library loads, exports every entry
point include/csa2.h declares, and rejects bad arguments on the host before
any HIP call (so these run on the CPU).  Also checks that the oracle and the
GPU library share no source."""
import ctypes
import os
import re

import pytest
import torch

import sparse_attention_fp4_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = csa2.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(csa2.EXPORTS)


def test_abi_version_and_status_strings():
    L = csa2.lib()
    assert L.csa2_abi_version() == 2 == csa2.ABI_VERSION
    for code, name in csa2.STATUS.items():
        assert L.csa2_status_string(code).decode() == name
    assert L.csa2_status_string(99).decode() == "CSA2_ERR_UNKNOWN"
    # the header's enum and the binding's table agree
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    enum = dict((int(v), k) for k, v in re.findall(r"\b(CSA2_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    assert enum == csa2.STATUS


def test_debug_build_exports_the_same_abi():
    from sparse_attention_fp4_amd.build import LIB_DEBUG
    D = csa2.load(LIB_DEBUG)
    for n in declared_functions():
        assert hasattr(D, n), n
    assert D.csa2_abi_version() == csa2.ABI_VERSION
    # host validation is the release build's
    assert D.csa2_index_full(*full_args(K=0)) == 2


V = ctypes.c_void_p
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails first


def err(rc):
    return rc, csa2.lib().csa2_last_error().decode()


def test_quantize_append_validation():
    L = csa2.lib()
    assert err(L.csa2_quantize_append(FAKE, 1, 4, 24, FAKE, FAKE, FAKE, 10, None))[0] == 2
    assert err(L.csa2_quantize_append(FAKE, 1, -1, 32, FAKE, FAKE, FAKE, 10, None))[0] == 2
    assert err(L.csa2_quantize_append(FAKE, 7, 4, 32, FAKE, FAKE, FAKE, 10, None))[0] == 3
    assert err(L.csa2_quantize_append(FAKE, 1, 4, 16384, FAKE, FAKE, FAKE, 10, None))[0] == 3
    assert err(L.csa2_quantize_append(None, 1, 4, 32, FAKE, FAKE, FAKE, 10, None))[0] == 1
    assert err(L.csa2_quantize_append(FAKE, 1, 4, 32, FAKE, FAKE, None, 10, None))[0] == 1
    # T == 0 is a no-op that succeeds without touching anything
    assert L.csa2_quantize_append(None, 1, 0, 32, None, None, None, 10, None) == 0


def full_args(**kw):
    a = dict(qI=FAKE, w=FAKE, ikeys=FAKE, ss=FAKE, rs=FAKE, rl=FAKE, R=2, Hi=64, Di=128, max_len=100,
             K=512, P=2048, block=8, topk=FAKE, pool=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return [a[k] for k in ("qI", "w", "ikeys", "ss", "rs", "rl", "R", "Hi", "Di", "max_len", "K", "P",
                           "block", "topk", "pool", "ws", "wsb")] + [None]


def test_index_full_validation():
    L = csa2.lib()
    f = L.csa2_index_full
    assert f(*full_args(K=0)) == 2
    assert f(*full_args(K=4096)) == 3
    assert f(*full_args(P=4096)) == 3
    assert f(*full_args(P=0)) == 2                  # pool given but P == 0
    assert f(*full_args(pool=None)) == 2            # P > 0 but no pool
    assert f(*full_args(Hi=0)) == 2
    assert f(*full_args(Hi=65)) == 3
    assert f(*full_args(Di=24)) == 2
    assert f(*full_args(Di=48)) == 3
    assert f(*full_args(Di=512)) == 3
    assert f(*full_args(block=4)) == 3
    assert f(*full_args(block=0)) == 2
    assert f(*full_args(max_len=-1)) == 2
    assert f(*full_args(R=-1)) == 2
    assert f(*full_args(qI=None)) == 1
    assert f(*full_args(topk=None)) == 1
    assert f(*full_args(wsb=16)) == 4
    assert f(*full_args(ws=None)) == 4
    assert f(*full_args(ws=ctypes.c_void_p(0x1001))) == 4      # misaligned
    assert "workspace" in csa2.lib().csa2_last_error().decode()
    assert f(*full_args(R=0)) == 0                              # empty batch: nothing to do


def test_index_full_workspace_formula():
    L = csa2.lib()
    # scores padded to 1024 entries per row plus block maxima, each 256-byte aligned
    assert L.csa2_index_full_workspace_bytes(32, 65536, 64, 512, 2048, 8) == 32 * 65536 * 4 + 32 * 8192 * 4
    assert L.csa2_index_full_workspace_bytes(1, 1, 1, 64, 256, 8) == 4096 + 512
    assert L.csa2_index_full_workspace_bytes(-1, 1, 1, 1, 1, 8) == 0


def test_index_reindex_workspace_formula():
    L = csa2.lib()
    # one fp32 score per pool slot, rows padded to whole scoring chunks
    assert L.csa2_index_reindex_workspace_bytes(32, 64, 512, 2048, 8) == 32 * 16384 * 4
    assert L.csa2_index_reindex_workspace_bytes(-1, 64, 512, 2048, 8) == 0


def reindex_args(**kw):
    a = dict(qI=FAKE, w=FAKE, ikeys=FAKE, ss=FAKE, rs=FAKE, rl=FAKE, pool=FAKE, R=2, Hi=64, Di=128,
             K=512, P=2048, block=8, topk=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return [a[k] for k in ("qI", "w", "ikeys", "ss", "rs", "rl", "pool", "R", "Hi", "Di", "K", "P",
                           "block", "topk", "ws", "wsb")] + [None]


def test_index_reindex_validation():
    f = csa2.lib().csa2_index_reindex
    assert f(*reindex_args(P=0)) == 2
    assert f(*reindex_args(P=3000)) == 3
    assert f(*reindex_args(K=0)) == 2
    assert f(*reindex_args(pool=None)) == 1
    assert f(*reindex_args(wsb=10)) == 4
    assert f(*reindex_args(R=0)) == 0


def attn_args(**kw):
    a = dict(q=FAKE, codes=FAKE, scales=FAKE, ss=FAKE, rs=FAKE, rl=FAKE, topk=FAKE, K=512, swa=FAKE,
             srs=FAKE, sl=FAKE, R=32, H=64, D=512, W=128, scale=0.04, out=FAKE, lse=None, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return [a[k] for k in ("q", "codes", "scales", "ss", "rs", "rl", "topk", "K", "swa", "srs", "sl", "R",
                           "H", "D", "W", "scale", "out", "lse", "ws", "wsb")] + [None]


def test_sparse_attn_validation():
    f = csa2.lib().csa2_sparse_attn
    assert f(*attn_args(D=96)) == 3
    assert f(*attn_args(D=64)) == 3
    assert f(*attn_args(D=40)) == 2
    assert f(*attn_args(H=0)) == 2
    assert f(*attn_args(K=-1)) == 2
    assert f(*attn_args(W=5000)) == 3
    assert f(*attn_args(topk=None)) == 1
    assert f(*attn_args(swa=None)) == 1
    assert f(*attn_args(out=None)) == 1
    assert f(*attn_args(R=2, wsb=0)) == 4   # few rows: split keys need a workspace
    assert f(*attn_args(R=0)) == 0


def test_sparse_attn_fp4mma_validation():
    """The native-FP4 form validates its arguments as csa2_sparse_attn does
    (its extra counter pointer may be NULL)."""
    f = csa2.lib().csa2_sparse_attn_fp4mma

    def args(**kw):
        a = attn_args(**kw)
        return a[:18] + [None] + a[18:]   # native_fragments after lse
    assert f(*args(D=96)) == 3
    assert f(*args(D=40)) == 2
    assert f(*args(H=0)) == 2
    assert f(*args(K=-1)) == 2
    assert f(*args(topk=None)) == 1
    assert f(*args(out=None)) == 1
    assert f(*args(R=2, wsb=0)) == 4
    assert f(*args(R=0)) == 0


def test_attn_workspace_only_when_split():
    L = csa2.lib()
    # many rows: one workgroup per (row, head group) fills the GPU -> no split, no workspace
    assert L.csa2_sparse_attn_workspace_bytes(4096, 64, 512, 512, 128) == 0
    # few rows: keys split across workgroups -> partial outputs need a workspace
    assert L.csa2_sparse_attn_workspace_bytes(2, 64, 512, 512, 128) > 0


def full_paged_args(**kw):
    a = dict(qI=FAKE, w=FAKE, ikeys=FAKE, rows=1 << 20, bt=FAKE, mp=64, pr=64, rs=FAKE, rl=FAKE, R=2, Hi=64,
             Di=128, max_len=100, K=512, P=2048, block=8, topk=FAKE, trows=None, pool=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return [a[k] for k in ("qI", "w", "ikeys", "rows", "bt", "mp", "pr", "rs", "rl", "R", "Hi", "Di", "max_len",
                           "K", "P", "block", "topk", "trows", "pool", "ws", "wsb")] + [None]


def reindex_paged_args(**kw):
    a = dict(qI=FAKE, w=FAKE, ikeys=FAKE, rows=1 << 20, bt=FAKE, mp=64, pr=64, rs=FAKE, rl=FAKE, pool=FAKE, R=2,
             Hi=64, Di=128, K=512, P=2048, block=8, topk=FAKE, trows=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return [a[k] for k in ("qI", "w", "ikeys", "rows", "bt", "mp", "pr", "rs", "rl", "pool", "R", "Hi", "Di",
                           "K", "P", "block", "topk", "trows", "ws", "wsb")] + [None]


@pytest.mark.parametrize("which", ["full", "reindex"])
def test_index_paged_validation(which):
    L = csa2.lib()
    f, args = ((L.csa2_index_full_paged, full_paged_args) if which == "full"
               else (L.csa2_index_reindex_paged, reindex_paged_args))
    assert f(*args(pr=48)) == 3                     # page_rows not a power of two
    assert f(*args(pr=4)) == 3                      # below 8 rows per page
    assert f(*args(pr=1 << 21)) == 3
    assert "page_rows" in L.csa2_last_error().decode()
    assert f(*args(mp=0)) == 2
    assert f(*args(rows=0)) == 2
    assert f(*args(bt=None)) == 1
    assert f(*args(K=0)) == 2                       # the packed call's own checks still apply
    assert f(*args(Hi=65)) == 3
    assert f(*args(wsb=16)) == 4
    assert f(*args(R=0, bt=None, pr=3)) == 0        # empty batch: nothing to check or do


def test_paged_rows_validation():
    f = csa2.lib().csa2_paged_rows
    ok = dict(bt=FAKE, mp=64, pr=64, rows=1 << 20, rs=FAKE, rl=FAKE, idx=FAKE, R=4, K=512, phys=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*[a[k] for k in ("bt", "mp", "pr", "rows", "rs", "rl", "idx", "R", "K", "phys")], None)

    assert call(pr=100) == 3
    assert call(mp=0) == 2
    assert call(rows=0) == 2
    assert call(R=-1) == 2
    assert call(idx=None) == 1
    assert call(phys=None) == 1
    assert call(R=0, idx=None, phys=None) == 0


def test_sparse_attn_phys_validation():
    f = csa2.lib().csa2_sparse_attn_phys
    ok = dict(q=FAKE, codes=FAKE, scales=FAKE, rows=1 << 20, idx=FAKE, K=512, swa=FAKE, srs=FAKE, sl=FAKE,
              head=None, R=32, H=64, D=512, W=128, scale=0.04, out=FAKE, lse=None, ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = dict(ok, **kw)
        return f(*[a[k] for k in ("q", "codes", "scales", "rows", "idx", "K", "swa", "srs", "sl", "head", "R",
                                  "H", "D", "W", "scale", "out", "lse", "ws", "wsb")], None)

    assert call(rows=0) == 2
    assert call(K=5000) == 3
    assert call(D=96) == 3
    assert call(idx=None) == 1
    assert call(swa=None) == 1
    assert call(out=None) == 1
    assert call(R=2, wsb=0) == 4
    assert call(R=0) == 0


def test_python_binding_rejects_host_tensors():
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        csa2.csa2_quantize_append(x, torch.zeros(4, dtype=torch.int64), torch.zeros(4, 16, dtype=torch.uint8),
                                  torch.zeros(4, 2, dtype=torch.uint8))


def test_oracle_and_library_share_no_source():
    pkg = os.path.join(ROOT, "sparse_attention_fp4_amd")
    lib_src = []
    for d, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".hip", ".h", ".py", ".cpp")):
                lib_src.append(open(os.path.join(d, f), encoding="utf-8").read())
    for s in lib_src:
        assert "import oracle" not in s and "from oracle" not in s and "csa2_oracle" not in s
    orc = open(os.path.join(ROOT, "oracle", "csa2_oracle.c"), encoding="utf-8").read()
    assert "#include \"" not in orc          # only system headers
    for d, _, files in os.walk(os.path.join(ROOT, "oracle")):
        for f in files:
            if f.endswith(".py"):
                s = open(os.path.join(d, f), encoding="utf-8").read()
                assert "sparse_attention_fp4_amd" not in s
