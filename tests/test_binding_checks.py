"""The Python binding checks every tensor it passes through the C ABI before
any call: dtypes, shapes (inputs and caller-provided outputs, which the C ABI
cannot size-check), contiguity, then that all of them live on one GPU.  Shape
checks come first, so these tests run on the CPU: a tensor of a wrong shape is
reported as such, and correctly shaped host tensors fail only the device
check."""
import pytest
import torch

import sparse_attention_fp4_amd as csa2

R, Hi, Di, K, P, H, D, W, ROWS = 3, 4, 64, 8, 4, 2, 128, 16, 100


def i32(*s):
    return torch.zeros(*s, dtype=torch.int32)


def index_inputs():
    return dict(qI=torch.zeros(R, Hi, Di, dtype=torch.uint8), w=torch.zeros(R, Hi),
                ikeys=torch.zeros(ROWS, Di, dtype=torch.uint8), seq_start=torch.zeros(1, dtype=torch.int64),
                row_seq=i32(R), row_len=i32(R))


def attn_inputs():
    return dict(q=torch.zeros(R, H, D, dtype=torch.bfloat16), codes=torch.zeros(ROWS, D // 2, dtype=torch.uint8),
                scales=torch.zeros(ROWS, D // 16, dtype=torch.uint8), seq_start=torch.zeros(1, dtype=torch.int64),
                row_seq=i32(R), row_len=i32(R), topk_idx=i32(R, K), swa=torch.zeros(ROWS, D, dtype=torch.uint8),
                swa_row_start=torch.zeros(R, dtype=torch.int64), swa_len=i32(R))


def full(**kw):
    a = index_inputs()
    return csa2.csa2_index_full(a["qI"], a["w"], a["ikeys"], a["seq_start"], a["row_seq"], a["row_len"], 100, K, P,
                                **kw)


def reindex(pool=None, **kw):
    a = index_inputs()
    return csa2.csa2_index_reindex(a["qI"], a["w"], a["ikeys"], a["seq_start"], a["row_seq"], a["row_len"],
                                   i32(R, P) if pool is None else pool, K, **kw)


def attn(**kw):
    a = attn_inputs()
    return csa2.csa2_sparse_attn(a["q"], a["codes"], a["scales"], a["seq_start"], a["row_seq"], a["row_len"],
                                 a["topk_idx"], a["swa"], a["swa_row_start"], a["swa_len"], W, 0.1, **kw)


def attn_fp4mma(**kw):
    a = attn_inputs()
    return csa2.csa2_sparse_attn_fp4mma(a["q"], a["codes"], a["scales"], a["seq_start"], a["row_seq"],
                                        a["row_len"], a["topk_idx"], a["swa"], a["swa_row_start"], a["swa_len"], W,
                                        0.1, **kw)


def attn_phys(**kw):
    a = attn_inputs()
    return csa2.csa2_sparse_attn_phys(a["q"], a["codes"], a["scales"], a["topk_idx"], a["swa"], a["swa_row_start"],
                                      a["swa_len"], W, 0.1, **kw)


def test_correct_shapes_on_the_host_fail_only_the_device_check():
    for call in (full, reindex, attn, attn_phys, attn_fp4mma):
        with pytest.raises(ValueError, match="must live on the GPU"):
            call()


@pytest.mark.parametrize("kw", [dict(topk_idx=i32(R, K + 1)), dict(topk_idx=i32(R + 1, K)), dict(topk_idx=i32(R * K)),
                                dict(pool_blocks=i32(R, P - 1)), dict(pool_blocks=i32(R - 1, P))])
def test_index_full_output_shapes(kw):
    with pytest.raises(ValueError, match="must have shape"):
        full(**kw)


def test_index_full_output_dtypes_and_layout():
    with pytest.raises(TypeError, match="int32"):
        full(topk_idx=torch.zeros(R, K, dtype=torch.int64))
    with pytest.raises(TypeError, match="int32"):
        full(pool_blocks=torch.zeros(R, P, dtype=torch.int64))
    with pytest.raises(ValueError, match="contiguous"):
        full(topk_idx=i32(K, R).t())


def test_index_reindex_shapes():
    with pytest.raises(ValueError, match="must have shape"):
        reindex(topk_idx=i32(R, K - 1))
    with pytest.raises(ValueError, match="pool_blocks must have shape"):
        reindex(pool=i32(R + 1, P))
    with pytest.raises(TypeError, match="int32"):
        reindex(pool=torch.zeros(R, P, dtype=torch.int64))


@pytest.mark.parametrize("call", [attn, attn_phys, attn_fp4mma])
def test_attention_output_shapes(call):
    with pytest.raises(ValueError, match="out must have shape"):
        call(out=torch.zeros(R, H, D - 16))
    with pytest.raises(ValueError, match="out must have shape"):
        call(out=torch.zeros(R * H, D))
    with pytest.raises(TypeError, match="float32"):
        call(out=torch.zeros(R, H, D, dtype=torch.float16))
    with pytest.raises(ValueError, match="lse must have shape"):
        call(lse=torch.zeros(R, H + 1))
    with pytest.raises(TypeError, match="float32"):
        call(lse=torch.zeros(R, H, dtype=torch.float64))


def test_attention_input_shapes():
    a = attn_inputs()
    with pytest.raises(ValueError, match="scales must have shape"):
        csa2.csa2_sparse_attn(a["q"], a["codes"], torch.zeros(ROWS + 1, D // 16, dtype=torch.uint8), a["seq_start"],
                              a["row_seq"], a["row_len"], a["topk_idx"], a["swa"], a["swa_row_start"], a["swa_len"],
                              W, 0.1)
    with pytest.raises(ValueError, match="topk_idx must have shape"):
        csa2.csa2_sparse_attn(a["q"], a["codes"], a["scales"], a["seq_start"], a["row_seq"], a["row_len"],
                              i32(R + 1, K), a["swa"], a["swa_row_start"], a["swa_len"], W, 0.1)
    with pytest.raises(ValueError, match="swa_len must have shape"):
        csa2.csa2_sparse_attn(a["q"], a["codes"], a["scales"], a["seq_start"], a["row_seq"], a["row_len"],
                              a["topk_idx"], a["swa"], a["swa_row_start"], i32(R + 2), W, 0.1)


def test_paged_outputs():
    a = index_inputs()
    bt = i32(1, 4)
    with pytest.raises(ValueError, match="topk_rows must have shape"):
        csa2.csa2_index_full_paged(a["qI"], a["w"], a["ikeys"], bt, 64, a["row_seq"], a["row_len"], 100, K, P,
                                   topk_rows=i32(R, K + 1))
    with pytest.raises(ValueError, match="pool_blocks must have shape"):
        csa2.csa2_index_full_paged(a["qI"], a["w"], a["ikeys"], bt, 64, a["row_seq"], a["row_len"], 100, K, P,
                                   pool_blocks=i32(R, P + 1))
    with pytest.raises(ValueError, match="phys must have shape"):
        csa2.csa2_paged_rows(bt, 64, ROWS, a["row_seq"], a["row_len"], i32(R, K), phys=i32(R, K - 1))
    idx = i32(R, K)
    with pytest.raises(ValueError, match="alias"):
        csa2.csa2_paged_rows(bt, 64, ROWS, a["row_seq"], a["row_len"], idx, phys=idx)


def test_quantize_shapes():
    x = torch.zeros(4, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dst_row must have shape"):
        csa2.csa2_quantize_append(x, torch.zeros(5, dtype=torch.int64), torch.zeros(8, D // 2, dtype=torch.uint8),
                                  torch.zeros(8, D // 16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales must have shape"):
        csa2.csa2_quantize_append(x, torch.zeros(4, dtype=torch.int64), torch.zeros(8, D // 2, dtype=torch.uint8),
                                  torch.zeros(7, D // 16, dtype=torch.uint8))


def test_fp4mma_counter_shape_and_dtype():
    with pytest.raises(ValueError, match="native_fragments must have shape"):
        attn_fp4mma(native_fragments=i32(2))
    with pytest.raises(TypeError, match="int32"):
        attn_fp4mma(native_fragments=torch.zeros(1, dtype=torch.int64))
