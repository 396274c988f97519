"""Python binding of the CSA2 HIP library (libcsa2.so) for MI355X / gfx950.

Argument marshalling only: every step of the hot path runs in the HIP kernels
behind the C ABI declared in include/csa2.h.  The functions below carry the
same names as the C entry points; they take torch tensors that live on the
GPU, check dtypes/shapes/contiguity, allocate outputs and workspaces when the
caller does not pass them, and enqueue the call on torch's current stream.

If the shared library has not been built, importing works but every call
raises RuntimeError: there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

CSA2_F32, CSA2_BF16 = 0, 1
STATUS = {0: "CSA2_OK", 1: "CSA2_ERR_NULL", 2: "CSA2_ERR_SHAPE", 3: "CSA2_ERR_UNSUPPORTED",
          4: "CSA2_ERR_WORKSPACE", 5: "CSA2_ERR_LAUNCH"}
EXPORTS = ("csa2_status_string", "csa2_last_error", "csa2_abi_version", "csa2_quantize_append",
           "csa2_index_full_workspace_bytes", "csa2_index_full",
           "csa2_index_reindex_workspace_bytes", "csa2_index_reindex",
           "csa2_sparse_attn_workspace_bytes", "csa2_sparse_attn",
           "csa2_index_full_paged", "csa2_index_reindex_paged", "csa2_paged_rows", "csa2_sparse_attn_phys")

_lib = None


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libcsa2.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sparse_attention_fp4_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.csa2_status_string.argtypes = [ctypes.c_int]
        L.csa2_status_string.restype = ctypes.c_char_p
        L.csa2_last_error.argtypes = []
        L.csa2_last_error.restype = ctypes.c_char_p
        L.csa2_abi_version.restype = ctypes.c_int
        L.csa2_quantize_append.argtypes = [P, i32, i32, i32, P, P, P, i64, P]
        L.csa2_index_full_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.csa2_index_full_workspace_bytes.restype = sz
        L.csa2_index_full.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, P, P, P, sz, P]
        L.csa2_index_reindex_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.csa2_index_reindex_workspace_bytes.restype = sz
        L.csa2_index_reindex.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, P, P, sz, P]
        L.csa2_sparse_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        L.csa2_sparse_attn_workspace_bytes.restype = sz
        L.csa2_sparse_attn.argtypes = [P, P, P, P, P, P, P, i32, P, P, P, i32, i32, i32, i32, f32, P, P, P,
                                       sz, P]
        L.csa2_index_full_paged.argtypes = [P, P, P, i64, P, i32, i32, P, P, i32, i32, i32, i32, i32, i32, i32,
                                            P, P, P, P, sz, P]
        L.csa2_index_reindex_paged.argtypes = [P, P, P, i64, P, i32, i32, P, P, P, i32, i32, i32, i32, i32, i32, P,
                                               P, P, sz, P]
        L.csa2_paged_rows.argtypes = [P, i32, i32, i64, P, P, P, i32, i32, P, P]
        L.csa2_sparse_attn_phys.argtypes = [P, P, P, i64, P, i32, P, P, P, P, i32, i32, i32, i32, f32, P, P, P,
                                            sz, P]
        for f in ("csa2_quantize_append", "csa2_index_full", "csa2_index_reindex", "csa2_sparse_attn",
                  "csa2_index_full_paged", "csa2_index_reindex_paged", "csa2_paged_rows", "csa2_sparse_attn_phys"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Csa2Error(fn, status, lib().csa2_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace holds {ws.numel() * ws.element_size()} bytes, needs {nbytes}")
    return ws


def _u8(t: torch.Tensor) -> torch.Tensor:
    """E4M3 tensors may be passed as torch.float8_e4m3fn or uint8 bit patterns."""
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


# ----------------------------------------------------------------------- a1

def csa2_quantize_append(x: torch.Tensor, dst_row: torch.Tensor, codes: torch.Tensor,
                         scales: torch.Tensor, stream=None) -> None:
    """Quantize rows x [T, D] (float32 or bfloat16) into cache rows dst_row [T]
    of codes [rows, D/2] uint8 and scales [rows, D/16] uint8 (E4M3)."""
    _dev(x, "x", None, 2)
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    T, D = x.shape
    _dev(dst_row, "dst_row", torch.int64, 1)
    _dev(codes, "codes", torch.uint8, 2)
    _dev(scales, "scales", torch.uint8, 2)
    if dst_row.shape[0] != T or codes.shape[1] * 2 != D or scales.shape[1] * 16 != D \
            or codes.shape[0] != scales.shape[0]:
        raise ValueError("shape mismatch between x, dst_row, codes and scales")
    st = lib().csa2_quantize_append(_ptr(x), CSA2_F32 if x.dtype == torch.float32 else CSA2_BF16,
                                    T, D, _ptr(dst_row), _ptr(codes), _ptr(scales), codes.shape[0],
                                    _stream(stream))
    _check("csa2_quantize_append", st)


# ----------------------------------------------------------------------- a2 + a3

def csa2_index_full_workspace_bytes(R: int, max_len: int, K: int, P: int, block: int = 8) -> int:
    return int(lib().csa2_index_full_workspace_bytes(R, max_len, K, P, block))


def csa2_index_full(qI: torch.Tensor, w: torch.Tensor, ikeys: torch.Tensor, seq_start: torch.Tensor,
                    row_seq: torch.Tensor, row_len: torch.Tensor, max_len: int, K: int, P: int,
                    block: int = 8, topk_idx: Optional[torch.Tensor] = None,
                    pool_blocks: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                    want_pool: bool = True, stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Full-mode indexer: returns (topk_idx [R, K], pool_blocks [R, P] or None)."""
    qI = _dev(_u8(qI), "qI", torch.uint8, 3)
    R, Hi, Di = qI.shape
    _dev(w, "w", torch.float32, 2)
    ikeys = _dev(_u8(ikeys), "ikeys", torch.uint8, 2)
    _dev(seq_start, "seq_start", torch.int64, 1)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    if tuple(w.shape) != (R, Hi) or ikeys.shape[1] != Di or row_seq.shape[0] != R or row_len.shape[0] != R:
        raise ValueError("shape mismatch among qI, w, ikeys, row_seq, row_len")
    dev = qI.device
    if topk_idx is None:
        topk_idx = torch.empty(R, K, dtype=torch.int32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    if want_pool and P > 0 and pool_blocks is None:
        pool_blocks = torch.empty(R, P, dtype=torch.int32, device=dev)
    Pc = P if pool_blocks is not None else 0
    ws = _workspace(csa2_index_full_workspace_bytes(R, max_len, K, Pc, block), dev, workspace)
    st = lib().csa2_index_full(_ptr(qI), _ptr(w), _ptr(ikeys), _ptr(seq_start), _ptr(row_seq), _ptr(row_len),
                               R, Hi, Di, max_len, K, Pc, block, _ptr(topk_idx), _ptr(pool_blocks),
                               _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("csa2_index_full", st)
    return topk_idx, pool_blocks


# ----------------------------------------------------------------------- a4

def csa2_index_reindex_workspace_bytes(R: int, K: int, P: int, block: int = 8) -> int:
    return int(lib().csa2_index_reindex_workspace_bytes(R, K, P, block))


def csa2_index_reindex(qI: torch.Tensor, w: torch.Tensor, ikeys: torch.Tensor, seq_start: torch.Tensor,
                       row_seq: torch.Tensor, row_len: torch.Tensor, pool_blocks: torch.Tensor, K: int,
                       block: int = 8, topk_idx: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Reindex-mode rescoring of the pool: returns topk_idx [R, K]."""
    qI = _dev(_u8(qI), "qI", torch.uint8, 3)
    R, Hi, Di = qI.shape
    _dev(w, "w", torch.float32, 2)
    ikeys = _dev(_u8(ikeys), "ikeys", torch.uint8, 2)
    _dev(seq_start, "seq_start", torch.int64, 1)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    _dev(pool_blocks, "pool_blocks", torch.int32, 2)
    P = pool_blocks.shape[1]
    if tuple(w.shape) != (R, Hi) or ikeys.shape[1] != Di or pool_blocks.shape[0] != R:
        raise ValueError("shape mismatch among qI, w, ikeys, pool_blocks")
    dev = qI.device
    if topk_idx is None:
        topk_idx = torch.empty(R, K, dtype=torch.int32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    ws = _workspace(csa2_index_reindex_workspace_bytes(R, K, P, block), dev, workspace)
    st = lib().csa2_index_reindex(_ptr(qI), _ptr(w), _ptr(ikeys), _ptr(seq_start), _ptr(row_seq),
                                  _ptr(row_len), _ptr(pool_blocks), R, Hi, Di, K, P, block, _ptr(topk_idx),
                                  _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check("csa2_index_reindex", st)
    return topk_idx


# ----------------------------------------------------------------------- a5

def csa2_sparse_attn_workspace_bytes(R: int, H: int, D: int, K: int, W: int) -> int:
    return int(lib().csa2_sparse_attn_workspace_bytes(R, H, D, K, W))


def csa2_sparse_attn(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, seq_start: torch.Tensor,
                     row_seq: torch.Tensor, row_len: torch.Tensor, topk_idx: torch.Tensor,
                     swa: Optional[torch.Tensor], swa_row_start: Optional[torch.Tensor],
                     swa_len: Optional[torch.Tensor], W: int, softmax_scale: float,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     want_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse MQA over the selected FP4 entries plus the FP8 SWA window.
    q: [R, H, D] bfloat16.  Returns (out [R, H, D] float32, lse [R, H] or None)."""
    if q.dtype == torch.bfloat16:
        q = q.view(torch.int16)
    _dev(q, "q", torch.int16, 3)
    R, H, D = q.shape
    _dev(codes, "codes", torch.uint8, 2)
    _dev(scales, "scales", torch.uint8, 2)
    _dev(seq_start, "seq_start", torch.int64, 1)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    K = topk_idx.shape[1]
    if codes.shape[1] * 2 != D or scales.shape[1] * 16 != D or topk_idx.shape[0] != R:
        raise ValueError("shape mismatch among q, codes, scales, topk_idx")
    if W > 0:
        swa = _dev(_u8(swa), "swa", torch.uint8, 2)
        _dev(swa_row_start, "swa_row_start", torch.int64, 1)
        _dev(swa_len, "swa_len", torch.int32, 1)
        if swa.shape[1] != D:
            raise ValueError("swa rows must have D channels")
    dev = q.device
    if out is None:
        out = torch.empty(R, H, D, dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32, 3)
    if want_lse and lse is None:
        lse = torch.empty(R, H, dtype=torch.float32, device=dev)
    ws = _workspace(csa2_sparse_attn_workspace_bytes(R, H, D, K, W), dev, workspace)
    st = lib().csa2_sparse_attn(_ptr(q), _ptr(codes), _ptr(scales), _ptr(seq_start), _ptr(row_seq),
                                _ptr(row_len), _ptr(topk_idx), K, _ptr(swa if W > 0 else None),
                                _ptr(swa_row_start if W > 0 else None), _ptr(swa_len if W > 0 else None),
                                R, H, D, W, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("csa2_sparse_attn", st)
    return out, lse


# ----------------------------------------------------------------- paged cache

def _pages(block_table: torch.Tensor, page_rows: int) -> int:
    _dev(block_table, "block_table", torch.int32, 2)
    if page_rows < 8 or page_rows & (page_rows - 1):
        raise ValueError("page_rows must be a power of two >= 8")
    return block_table.shape[1]


def csa2_index_full_paged(qI: torch.Tensor, w: torch.Tensor, ikeys: torch.Tensor, block_table: torch.Tensor,
                          page_rows: int, row_seq: torch.Tensor, row_len: torch.Tensor, max_len: int, K: int,
                          P: int, block: int = 8, topk_idx: Optional[torch.Tensor] = None,
                          pool_blocks: Optional[torch.Tensor] = None, want_pool: bool = True,
                          topk_rows: Optional[torch.Tensor] = None, want_rows: bool = False,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """csa2_index_full over a paged key cache: entry j of sequence s is cache row
    block_table[s, j // page_rows] * page_rows + j % page_rows.  Returns
    (topk_idx, pool_blocks, topk_rows); topk_rows (the cache rows of the Top-K
    entries) is None unless given or want_rows."""
    qI = _dev(_u8(qI), "qI", torch.uint8, 3)
    R, Hi, Di = qI.shape
    _dev(w, "w", torch.float32, 2)
    ikeys = _dev(_u8(ikeys), "ikeys", torch.uint8, 2)
    max_pages = _pages(block_table, page_rows)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    if tuple(w.shape) != (R, Hi) or ikeys.shape[1] != Di or row_seq.shape[0] != R or row_len.shape[0] != R:
        raise ValueError("shape mismatch among qI, w, ikeys, row_seq, row_len")
    dev = qI.device
    if topk_idx is None:
        topk_idx = torch.empty(R, K, dtype=torch.int32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    if want_pool and P > 0 and pool_blocks is None:
        pool_blocks = torch.empty(R, P, dtype=torch.int32, device=dev)
    if want_rows and topk_rows is None:
        topk_rows = torch.empty(R, K, dtype=torch.int32, device=dev)
    if topk_rows is not None:
        _dev(topk_rows, "topk_rows", torch.int32, 2)
        if tuple(topk_rows.shape) != (R, K):
            raise ValueError("topk_rows must be [R, K]")
    Pc = P if pool_blocks is not None else 0
    ws = _workspace(csa2_index_full_workspace_bytes(R, max_len, K, Pc, block), dev, workspace)
    st = lib().csa2_index_full_paged(_ptr(qI), _ptr(w), _ptr(ikeys), ikeys.shape[0], _ptr(block_table), max_pages,
                                     page_rows, _ptr(row_seq), _ptr(row_len), R, Hi, Di, max_len, K, Pc, block,
                                     _ptr(topk_idx), _ptr(topk_rows), _ptr(pool_blocks), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("csa2_index_full_paged", st)
    return topk_idx, pool_blocks, topk_rows


def csa2_index_reindex_paged(qI: torch.Tensor, w: torch.Tensor, ikeys: torch.Tensor, block_table: torch.Tensor,
                             page_rows: int, row_seq: torch.Tensor, row_len: torch.Tensor,
                             pool_blocks: torch.Tensor, K: int, block: int = 8,
                             topk_idx: Optional[torch.Tensor] = None, topk_rows: Optional[torch.Tensor] = None,
                             want_rows: bool = False, workspace: Optional[torch.Tensor] = None,
                             stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """csa2_index_reindex over a paged key cache (addressing as
    csa2_index_full_paged).  Returns (topk_idx, topk_rows)."""
    qI = _dev(_u8(qI), "qI", torch.uint8, 3)
    R, Hi, Di = qI.shape
    _dev(w, "w", torch.float32, 2)
    ikeys = _dev(_u8(ikeys), "ikeys", torch.uint8, 2)
    max_pages = _pages(block_table, page_rows)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    _dev(pool_blocks, "pool_blocks", torch.int32, 2)
    P = pool_blocks.shape[1]
    if tuple(w.shape) != (R, Hi) or ikeys.shape[1] != Di or pool_blocks.shape[0] != R:
        raise ValueError("shape mismatch among qI, w, ikeys, pool_blocks")
    dev = qI.device
    if topk_idx is None:
        topk_idx = torch.empty(R, K, dtype=torch.int32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    if want_rows and topk_rows is None:
        topk_rows = torch.empty(R, K, dtype=torch.int32, device=dev)
    if topk_rows is not None:
        _dev(topk_rows, "topk_rows", torch.int32, 2)
        if tuple(topk_rows.shape) != (R, K):
            raise ValueError("topk_rows must be [R, K]")
    ws = _workspace(csa2_index_reindex_workspace_bytes(R, K, P, block), dev, workspace)
    st = lib().csa2_index_reindex_paged(_ptr(qI), _ptr(w), _ptr(ikeys), ikeys.shape[0], _ptr(block_table),
                                        max_pages, page_rows, _ptr(row_seq), _ptr(row_len), _ptr(pool_blocks), R,
                                        Hi, Di, K, P, block, _ptr(topk_idx), _ptr(topk_rows), _ptr(ws),
                                        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("csa2_index_reindex_paged", st)
    return topk_idx, topk_rows


def csa2_paged_rows(block_table: torch.Tensor, page_rows: int, cache_rows: int, row_seq: torch.Tensor,
                    row_len: torch.Tensor, idx: torch.Tensor, phys: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """Cache rows [R, K] of the entries of index lists idx [R, K] over a paged cache (-1: none)."""
    max_pages = _pages(block_table, page_rows)
    _dev(row_seq, "row_seq", torch.int32, 1)
    _dev(row_len, "row_len", torch.int32, 1)
    _dev(idx, "idx", torch.int32, 2)
    R, K = idx.shape
    if row_seq.shape[0] != R or row_len.shape[0] != R:
        raise ValueError("shape mismatch among idx, row_seq, row_len")
    if phys is None:
        phys = torch.empty(R, K, dtype=torch.int32, device=idx.device)
    _dev(phys, "phys", torch.int32, 2)
    st = lib().csa2_paged_rows(_ptr(block_table), max_pages, page_rows, int(cache_rows), _ptr(row_seq),
                               _ptr(row_len), _ptr(idx), R, K, _ptr(phys), _stream(stream))
    _check("csa2_paged_rows", st)
    return phys


def csa2_sparse_attn_phys(q: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, phys_idx: torch.Tensor,
                          swa: Optional[torch.Tensor], swa_row_start: Optional[torch.Tensor],
                          swa_len: Optional[torch.Tensor], W: int, softmax_scale: float,
                          swa_head: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                          workspace: Optional[torch.Tensor] = None,
                          stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """csa2_sparse_attn over cache rows (phys_idx from csa2_paged_rows), with an
    optional SWA ring: window row i of row r in slot (swa_head[r] + i) % W."""
    if q.dtype == torch.bfloat16:
        q = q.view(torch.int16)
    _dev(q, "q", torch.int16, 3)
    R, H, D = q.shape
    _dev(codes, "codes", torch.uint8, 2)
    _dev(scales, "scales", torch.uint8, 2)
    _dev(phys_idx, "phys_idx", torch.int32, 2)
    K = phys_idx.shape[1]
    if codes.shape[1] * 2 != D or scales.shape[1] * 16 != D or phys_idx.shape[0] != R:
        raise ValueError("shape mismatch among q, codes, scales, phys_idx")
    if W > 0:
        swa = _dev(_u8(swa), "swa", torch.uint8, 2)
        _dev(swa_row_start, "swa_row_start", torch.int64, 1)
        _dev(swa_len, "swa_len", torch.int32, 1)
        if swa_head is not None:
            _dev(swa_head, "swa_head", torch.int32, 1)
        if swa.shape[1] != D:
            raise ValueError("swa rows must have D channels")
    dev = q.device
    if out is None:
        out = torch.empty(R, H, D, dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32, 3)
    if want_lse and lse is None:
        lse = torch.empty(R, H, dtype=torch.float32, device=dev)
    ws = _workspace(csa2_sparse_attn_workspace_bytes(R, H, D, K, W), dev, workspace)
    st = lib().csa2_sparse_attn_phys(_ptr(q), _ptr(codes), _ptr(scales), codes.shape[0], _ptr(phys_idx), K,
                                     _ptr(swa if W > 0 else None), _ptr(swa_row_start if W > 0 else None),
                                     _ptr(swa_len if W > 0 else None), _ptr(swa_head if W > 0 else None), R, H,
                                     D, W, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check("csa2_sparse_attn_phys", st)
    return out, lse
