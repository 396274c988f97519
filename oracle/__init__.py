"""CPU oracle for the CSA2 decode hot path — test infrastructure only.

The oracle is the plain C file ``csa2_oracle.c`` next to this module (fp64,
plain loops), loaded through ctypes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg import this package; the GPU library never
does, and the two share no code.  Everything here is argument marshalling from
numpy arrays to the C entry points.

Sources of what is computed: the blog teardown "DeepSeek V4.1 Flash 拆解"
(austincafe.tech), section 一 (CSA2 layer modes, Hierarchical Sparse Indexer,
FP4 KV cache), and the arXiv abstract of "DeepSeek-V4.1-Flash: Pushing the
Limits of KV Cache Compression".  The C file documents each reading.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libcsa2_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math) and return the path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.csa2_ref_e2m1_value.argtypes = [ctypes.c_int]
        L.csa2_ref_e2m1_value.restype = ctypes.c_double
        L.csa2_ref_e4m3_value.argtypes = [ctypes.c_int]
        L.csa2_ref_e4m3_value.restype = ctypes.c_double
        L.csa2_ref_e4m3_encode.argtypes = [ctypes.c_double]
        L.csa2_ref_e4m3_encode.restype = ctypes.c_int
        L.csa2_ref_quantize_append.argtypes = [P, ctypes.c_int, i32, i32, P, P, P, i64]
        L.csa2_ref_dequant_rows.argtypes = [P, P, i64, i32, P]
        L.csa2_ref_index_scores.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, P]
        L.csa2_ref_index_full.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32, P, P]
        L.csa2_ref_index_reindex.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, P]
        L.csa2_ref_sparse_attn.argtypes = [P, P, P, P, P, P, P, i32, P, P, P, i32, i32, i32, i32, f32,
                                      P, P, P]
        L.csa2_ref_dense_attn.argtypes = [P, P, P, P, P, P, P, P, i32, i32, i32, ctypes.c_double, P]
        for f in ("csa2_ref_quantize_append", "csa2_ref_dequant_rows", "csa2_ref_index_scores", "csa2_ref_index_full",
                  "csa2_ref_index_reindex", "csa2_ref_sparse_attn", "csa2_ref_dense_attn"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its inputs (code {rc})")


# ---------------------------------------------------------------- formats

def e2m1_value(code: int) -> float:
    return lib().csa2_ref_e2m1_value(int(code))


def e4m3_value(bits: int) -> float:
    return lib().csa2_ref_e4m3_value(int(bits))


def e4m3_encode(v: float) -> int:
    return lib().csa2_ref_e4m3_encode(float(v))


# ---------------------------------------------------------------- a1

def quantize_append(x: np.ndarray, dtype: str, dst_row: np.ndarray, codes: np.ndarray,
                    scales: np.ndarray) -> None:
    """x: [T, D] float32, or uint16 bf16 bit patterns when dtype == 'bf16'.
    Writes codes [rows, D/2] and scales [rows, D/16] (uint8) in place."""
    T, D = x.shape
    xd = _c(x, np.float32 if dtype == "f32" else np.uint16)
    dr = _c(dst_row, np.int64)
    assert codes.dtype == np.uint8 and scales.dtype == np.uint8
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    rc = lib().csa2_ref_quantize_append(_p(xd), 0 if dtype == "f32" else 1, T, D, _p(dr),
                                   _p(codes), _p(scales), codes.shape[0])
    _check(rc, "quantize_append")


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    rows, half = codes.shape
    D = half * 2
    out = np.empty((rows, D), np.float64)
    rc = lib().csa2_ref_dequant_rows(_p(_c(codes, np.uint8)), _p(_c(scales, np.uint8)), rows, D, _p(out))
    _check(rc, "dequant_rows")
    return out


# ---------------------------------------------------------------- a2 / a3 / a4

def index_scores(qI, w, ikeys, seq_start, row_seq, row_len, max_len):
    R, Hi, Di = qI.shape
    out = np.empty((R, max_len), np.float32)
    rc = lib().csa2_ref_index_scores(_p(_c(qI, np.uint8)), _p(_c(w, np.float32)), _p(_c(ikeys, np.uint8)),
                                _p(_c(seq_start, np.int64)), _p(_c(row_seq, np.int32)),
                                _p(_c(row_len, np.int32)), R, Hi, Di, max_len, _p(out))
    _check(rc, "index_scores")
    return out


def index_full(qI, w, ikeys, seq_start, row_seq, row_len, max_len, K, P, block=8, want_pool=True):
    R, Hi, Di = qI.shape
    topk = np.empty((R, K), np.int32)
    pool = np.empty((R, P), np.int32) if want_pool else None
    rc = lib().csa2_ref_index_full(_p(_c(qI, np.uint8)), _p(_c(w, np.float32)), _p(_c(ikeys, np.uint8)),
                              _p(_c(seq_start, np.int64)), _p(_c(row_seq, np.int32)),
                              _p(_c(row_len, np.int32)), R, Hi, Di, max_len, K, P, block,
                              _p(topk), _p(pool))
    _check(rc, "index_full")
    return topk, pool


def index_reindex(qI, w, ikeys, seq_start, row_seq, row_len, pool, K, block=8):
    R, Hi, Di = qI.shape
    P = pool.shape[1]
    topk = np.empty((R, K), np.int32)
    rc = lib().csa2_ref_index_reindex(_p(_c(qI, np.uint8)), _p(_c(w, np.float32)), _p(_c(ikeys, np.uint8)),
                                 _p(_c(seq_start, np.int64)), _p(_c(row_seq, np.int32)),
                                 _p(_c(row_len, np.int32)), _p(_c(pool, np.int32)), R, Hi, Di,
                                 K, P, block, _p(topk))
    _check(rc, "index_reindex")
    return topk


# ---------------------------------------------------------------- a5

def sparse_attn(q_bits, codes, scales, seq_start, row_seq, row_len, topk_idx, swa,
                swa_row_start, swa_len, W, softmax_scale, rows=None, want_lse=True):
    """q_bits: [R, H, D] uint16 (bf16 patterns).  Returns (out [R,H,D] f32,
    lse [R,H] f32).  `rows` (iterable of row ids) limits the rows computed;
    the others are NaN."""
    R, H, D = q_bits.shape
    K = topk_idx.shape[1]
    out = np.full((R, H, D), np.nan, np.float32)
    lse = np.full((R, H), np.nan, np.float32) if want_lse else None
    mask = None
    if rows is not None:
        mask = np.zeros(R, np.uint8)
        mask[np.asarray(list(rows), dtype=np.int64)] = 1
    rc = lib().csa2_ref_sparse_attn(_p(_c(q_bits, np.uint16)), _p(_c(codes, np.uint8)), _p(_c(scales, np.uint8)),
                               _p(_c(seq_start, np.int64)), _p(_c(row_seq, np.int32)),
                               _p(_c(row_len, np.int32)), _p(_c(topk_idx, np.int32)), K,
                               _p(_c(swa, np.uint8)), _p(_c(swa_row_start, np.int64)),
                               _p(_c(swa_len, np.int32)), R, H, D, W, float(softmax_scale),
                               _p(out), _p(lse), _p(mask))
    _check(rc, "sparse_attn")
    return out, lse


def dense_attn(q_bits, kv_vals, seq_start, row_seq, row_len, swa_vals, swa_row_start, swa_len,
               softmax_scale):
    R, H, D = q_bits.shape
    out = np.empty((R, H, D), np.float64)
    rc = lib().csa2_ref_dense_attn(_p(_c(q_bits, np.uint16)), _p(_c(kv_vals, np.float64)),
                              _p(_c(seq_start, np.int64)), _p(_c(row_seq, np.int32)),
                              _p(_c(row_len, np.int32)), _p(_c(swa_vals, np.float64)),
                              _p(_c(swa_row_start, np.int64)), _p(_c(swa_len, np.int32)),
                              R, H, D, float(softmax_scale), _p(out))
    _check(rc, "dense_attn")
    return out
