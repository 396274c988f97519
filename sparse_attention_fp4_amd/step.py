"""CSA2 layer schedule: one decode (or prefill-chunk) step over the C ABI.

Section 一 of the teardown "DeepSeek V4.1 Flash 拆解" (austincafe.tech) gives
the three layer modes: a Full layer runs its own indexer over every entry,
keeps a Top-K and builds the block pool; a Reindex layer rescores the pool with
its own indexer query and keeps its own Top-K; a Reuse layer attends with the
indices of an earlier layer.  Reading of the reuse link: a Reuse layer inherits
from the nearest preceding Full or Reindex layer, and every Reindex layer uses
the pool of the Full layer.

`CSA2Step` allocates every output and workspace once, so `run()` only enqueues
kernels (nothing is allocated, copied or synchronised inside a step).

Paged mode (block_table given): the main cache and the indexer keys are paged
caches addressed through the block table, new_rows are cache rows, the two
indexer calls take their paged forms and also write the cache rows of each
Full/Reindex layer's Top-K entries, and every attention call reads those rows.
With swa_head given the SWA window of each row is a ring of W slots.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from . import (csa2_index_full, csa2_index_full_paged, csa2_index_full_workspace_bytes, csa2_index_reindex,
               csa2_index_reindex_paged, csa2_index_reindex_workspace_bytes, csa2_quantize_append, csa2_sparse_attn, csa2_sparse_attn_phys, csa2_sparse_attn_workspace_bytes)


def parent_layers(modes: List[str]) -> List[int]:
    """For each layer, the layer whose Top-K list its attention uses."""
    out, last = [], None
    for l, m in enumerate(modes):
        if m not in "FRU":
            raise ValueError(f"unknown layer mode {m!r}")
        if m in "FR":
            last = l
        if last is None:
            raise ValueError("the first layer must be Full")
        if m == "R" and "F" not in modes[:l]:
            raise ValueError("a Reindex layer needs an earlier Full layer's pool")
        out.append(last)
    return out


class CSA2Step:
    """Buffers and launch sequence of one CSA2 step.

    Inputs (all CUDA tensors):
      codes, scales        main cache (FP4 codes, E4M3 scales)
      ikeys                indexer keys [rows, Di] E4M3
      seq_start, row_seq, row_len, max_len
      new_kv, new_rows     entries appended at the start of the step
      qI[l], w[l]          indexer query/weights of Full and Reindex layers
      q[l], swa[l]         attention query and SWA rows of every layer
      swa_row_start, swa_len, W
      block_table, page_rows   paged mode (seq_start unused)
      swa_head             SWA ring heads [R] int32 (paged mode only)
    """

    def __init__(self, modes: List[str], *, codes, scales, ikeys, seq_start, row_seq, row_len, max_len,
                 new_kv, new_rows, qI: Dict[int, torch.Tensor], w: Dict[int, torch.Tensor],
                 q: Dict[int, torch.Tensor], swa: Dict[int, torch.Tensor], swa_row_start, swa_len, W: int,
                 K: int, P: int, softmax_scale: float, block: int = 8, block_table=None, page_rows: int = 0,
                 swa_head=None):
        self.modes = list(modes)
        self.parents = parent_layers(self.modes)
        self.codes, self.scales, self.ikeys = codes, scales, ikeys
        self.seq_start, self.row_seq, self.row_len, self.max_len = seq_start, row_seq, row_len, int(max_len)
        self.new_kv, self.new_rows = new_kv, new_rows
        self.qI, self.w, self.q, self.swa = qI, w, q, swa
        self.swa_row_start, self.swa_len, self.W = swa_row_start, swa_len, int(W)
        self.K, self.P, self.block, self.scale = int(K), int(P), int(block), float(softmax_scale)
        self.block_table, self.page_rows, self.swa_head = block_table, int(page_rows), swa_head
        self.paged = block_table is not None
        if swa_head is not None and not self.paged:
            raise ValueError("swa_head needs paged mode")
        dev = codes.device
        R = int(row_seq.shape[0])
        H, D = q[0].shape[1], q[0].shape[2]
        self.R, self.H, self.D = R, H, D
        self.topk = {l: torch.empty(R, self.K, dtype=torch.int32, device=dev)
                     for l, m in enumerate(self.modes) if m in "FR"}
        self.pool = torch.empty(R, self.P, dtype=torch.int32, device=dev)
        self.phys = ({l: torch.empty(R, self.K, dtype=torch.int32, device=dev) for l in self.topk}
                     if self.paged else self.topk)
        self.out = {l: torch.empty(R, H, D, dtype=torch.float32, device=dev) for l in range(len(self.modes))}
        self.lse = {l: torch.empty(R, H, dtype=torch.float32, device=dev) for l in range(len(self.modes))}
        Hi = int(qI[self.modes.index("F")].shape[1])
        nbytes = max(csa2_index_full_workspace_bytes(R, self.max_len, Hi, self.K, self.P, self.block),
                     csa2_index_reindex_workspace_bytes(R, Hi, self.K, self.P, self.block), 256)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # the attention calls keep arrival words in theirs: zeroed once, left zero by every call
        self.attn_workspace = torch.zeros(max(csa2_sparse_attn_workspace_bytes(R, H, D, self.K, self.W), 256),
                                          dtype=torch.uint8, device=dev)

    def run(self, stream=None, layers=None, mark=None) -> None:
        """Enqueue the step.  `mark(label, phase)` (optional) is called right
        before ("begin") and after ("end") each library call, on the host, so a
        caller can record HIP events around individual calls."""
        def _mark(label, phase):
            if mark is not None:
                mark(label, phase)

        if self.new_kv is not None and self.new_kv.shape[0] > 0:
            _mark("quantize_append", "begin")
            csa2_quantize_append(self.new_kv, self.new_rows, self.codes, self.scales, stream=stream)
            _mark("quantize_append", "end")
        for l, m in enumerate(self.modes):
            if m == "F":
                _mark("index_full", "begin")
                if self.paged:
                    csa2_index_full_paged(self.qI[l], self.w[l], self.ikeys, self.block_table, self.page_rows,
                                          self.row_seq, self.row_len, self.max_len, self.K, self.P, self.block,
                                          topk_idx=self.topk[l], pool_blocks=self.pool, topk_rows=self.phys[l],
                                          workspace=self.workspace, stream=stream)
                else:
                    csa2_index_full(self.qI[l], self.w[l], self.ikeys, self.seq_start, self.row_seq, self.row_len,
                                    self.max_len, self.K, self.P, self.block, topk_idx=self.topk[l],
                                    pool_blocks=self.pool, workspace=self.workspace, stream=stream)
                _mark("index_full", "end")
            elif m == "R":
                _mark("index_reindex", "begin")
                if self.paged:
                    csa2_index_reindex_paged(self.qI[l], self.w[l], self.ikeys, self.block_table, self.page_rows,
                                             self.row_seq, self.row_len, self.pool, self.K, self.block,
                                             topk_idx=self.topk[l], topk_rows=self.phys[l], workspace=self.workspace,
                                             stream=stream)
                else:
                    csa2_index_reindex(self.qI[l], self.w[l], self.ikeys, self.seq_start, self.row_seq,
                                       self.row_len, self.pool, self.K, self.block, topk_idx=self.topk[l],
                                       workspace=self.workspace, stream=stream)
                _mark("index_reindex", "end")
            if layers is not None and l not in layers:
                continue
            _mark("sparse_attn", "begin")
            if self.paged:
                csa2_sparse_attn_phys(self.q[l], self.codes, self.scales, self.phys[self.parents[l]], self.swa[l],
                                      self.swa_row_start, self.swa_len, self.W, self.scale, swa_head=self.swa_head,
                                      out=self.out[l], lse=self.lse[l], workspace=self.attn_workspace,
                                      stream=stream)
            else:
                csa2_sparse_attn(self.q[l], self.codes, self.scales, self.seq_start, self.row_seq, self.row_len,
                                 self.topk[self.parents[l]], self.swa[l], self.swa_row_start, self.swa_len, self.W,
                                 self.scale, out=self.out[l], lse=self.lse[l], workspace=self.attn_workspace,
                                 stream=stream)
            _mark("sparse_attn", "end")
