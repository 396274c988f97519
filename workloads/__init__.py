"""Seeded synthetic workloads for the CSA2 decode hot path.

This module only draws random inputs; it holds none of the method's
arithmetic (no quantisation, scoring, selection or attention).  Both the GPU
library's tests/benchmark and the CPU oracle consume what it produces.
Casts to bfloat16 and FP8 E4M3 are torch's own conversions
(round-to-nearest-even), applied to values that the recipe keeps in range.

Shapes and distributions follow the five workloads the method is measured on
(tiny parity case, decode at 64K entries, decode at 1M entries, a 4096-token
prefill chunk against 131,072 entries, and a ragged heavy-tailed decode batch).
The pages fix none of the head counts or dims; the values below are the
stated choices.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

BASE_SEED = 20260917


@dataclasses.dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int                    # sequences
    N: Optional[int]          # entries per sequence (None = ragged)
    D: int                    # main KV latent dim
    W: int                    # SWA window
    H: int                    # attention query heads
    Hi: int                   # indexer heads
    Di: int                   # indexer dim
    K: int                    # Top-K
    P: int                    # pool blocks
    block: int = 8
    kv_dtype: str = "bf16"    # raw main-KV dtype fed to the quantizer
    kv_dist: str = "normal"   # "normal" | "student_t_outliers"
    idx_dist: str = "int3"    # "int3" (uniform integers in [-3,3]) | "ties"
    w_dist: str = "u01_16"    # "ones" | "u01_16" (U(0,1) rounded to 1/16)
    layers: str = "F" + "UUUU" + "R" + "UUUU" + "R" + "UUUU" + "R" + "UUUU"
    prefill_rows: int = 0     # >0: causal prefill chunk of that many rows
    ragged_lo: int = 0
    ragged_hi: int = 0

    @property
    def seed(self) -> int:
        return BASE_SEED + self.cid


CONFIGS = {
    1: Config(1, "tiny", B=1, N=4096, D=128, W=32, H=8, Hi=1, Di=64, K=64, P=256,
              kv_dtype="f32", w_dist="ones", layers="FRU"),
    2: Config(2, "decode_64k", B=32, N=65536, D=512, W=128, H=64, Hi=64, Di=128, K=512, P=2048),
    3: Config(3, "decode_1m", B=4, N=1048576, D=512, W=128, H=64, Hi=64, Di=128, K=512, P=2048),
    4: Config(4, "prefill_chunk", B=1, N=131072, D=512, W=128, H=64, Hi=64, Di=128, K=512, P=2048,
              layers="F", prefill_rows=4096),
    5: Config(5, "ragged_256", B=256, N=None, D=512, W=128, H=64, Hi=64, Di=128, K=512, P=2048,
              kv_dist="student_t_outliers", idx_dist="ties", ragged_lo=4096, ragged_hi=262144),
    # the prefill chunk of config 4 run through the decode layer schedule: every chunk row gets the
    # Full layer's pool, three pool-restricted Reindex layers and Reuse attention in the other layers
    6: Config(6, "prefill_layers", B=1, N=131072, D=512, W=128, H=64, Hi=64, Di=128, K=512, P=2048,
              prefill_rows=4096),
}


def layer_modes(cfg: Config) -> List[str]:
    """'F' Full, 'R' Reindex, 'U' Reuse per decoder layer (the chosen pattern)."""
    return list(cfg.layers)


def scaled(cfg: Config, **kw) -> Config:
    """A copy of a config with some sizes replaced (for small parity cases)."""
    return dataclasses.replace(cfg, **kw)


# ------------------------------------------------------------------ helpers

def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def to_e4m3_bytes(x: torch.Tensor) -> torch.Tensor:
    """torch's E4M3 cast (RNE) after clamping to +-448; returns uint8 bits."""
    return x.float().clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)


def bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def seq_lengths(cfg: Config) -> np.ndarray:
    if cfg.N is not None:
        n = np.full(cfg.B, cfg.N, np.int64)
        if cfg.prefill_rows:
            n = n + cfg.prefill_rows
        return n
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    u = rng.uniform(math.log(cfg.ragged_lo), math.log(cfg.ragged_hi), size=cfg.B)
    return np.floor(np.exp(u)).astype(np.int64)


def _int_values(cfg: Config, shape, g, device, alphabet=None) -> torch.Tensor:
    if cfg.idx_dist == "int3":
        return torch.randint(-3, 4, shape, generator=g, device=device).float()
    # "ties": values in {-1, 0, 1}; keys drawn from a small alphabet so that many
    # scores and block maxima repeat exactly
    if alphabet is not None:
        pick = torch.randint(0, alphabet.shape[0], shape[:-1], generator=g, device=device)
        return alphabet[pick]
    return torch.randint(-1, 2, shape, generator=g, device=device).float()


def _weights(cfg: Config, shape, g, device) -> torch.Tensor:
    if cfg.w_dist == "ones":
        return torch.ones(shape, device=device)
    return torch.round(torch.rand(shape, generator=g, device=device) * 16.0) / 16.0


def _kv_raw(cfg: Config, rows: int, g, device, outlier_ch) -> torch.Tensor:
    if cfg.kv_dist == "normal":
        x = torch.randn(rows, cfg.D, generator=g, device=device)
    else:
        # Student-t with 3 degrees of freedom: N(0,1) / sqrt(chi2_3 / 3)
        z = torch.randn(rows, cfg.D, generator=g, device=device)
        c = torch.randn(rows, cfg.D, 3, generator=g, device=device).pow_(2).sum(-1)
        x = z / torch.sqrt(c / 3.0)
        x[:, outlier_ch] *= 20.0
    return x if cfg.kv_dtype == "f32" else x.to(torch.bfloat16)


@dataclasses.dataclass
class Workload:
    cfg: Config
    lengths: np.ndarray            # [B] entries per sequence (after any append)
    seq_start: torch.Tensor        # [B] int64 first cache row of each sequence
    rows_total: int
    row_seq: torch.Tensor          # [R] int32
    row_len: torch.Tensor          # [R] int32 visible entries per query row
    kv_raw: torch.Tensor           # [rows_total, D] f32 or bf16 (pre-quantisation values)
    ikeys: torch.Tensor            # [rows_total, Di] uint8 E4M3
    qI: dict                       # layer -> [R, Hi, Di] uint8 (F and R layers)
    w: dict                        # layer -> [R, Hi] f32
    q: dict                        # layer -> [R, H, D] bf16
    swa: dict                      # layer -> [R*W (+extra), D] uint8 E4M3
    swa_row_start: torch.Tensor    # [R] int64
    swa_len: torch.Tensor          # [R] int32
    new_rows: Optional[torch.Tensor] = None   # cache rows the step appends (dst_row)

    @property
    def R(self) -> int:
        return int(self.row_seq.shape[0])


def make(cfg: Config, device="cpu", layers: Optional[List[int]] = None,
         lengths: Optional[np.ndarray] = None) -> Workload:
    """Draw every input of one step of `cfg` on `device` with the config's seed.

    Decode configs: one query row per sequence seeing all its entries; the last
    entry of each sequence is the one the step appends.  Prefill (configs 4, 6):
    the chunk's rows are appended after the 131,072 cached entries and query
    row i sees 131,072 + i + 1 entries; its SWA window is token rows
    [i, i + W) of one [W - 1 + rows, D] buffer.
    """
    g = _gen(cfg.seed, device)
    lengths = seq_lengths(cfg) if lengths is None else np.asarray(lengths, np.int64)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]]).astype(np.int64)
    rows_total = int(lengths.sum())
    modes = layer_modes(cfg)
    if layers is None:
        layers = list(range(len(modes)))

    outlier_ch = None
    if cfg.kv_dist != "normal":
        # 4 fixed channels per 16-channel group
        gg = np.random.Generator(np.random.PCG64(cfg.seed + 1000))
        ch = []
        for grp in range(cfg.D // 16):
            ch.extend(grp * 16 + gg.choice(16, 4, replace=False))
        outlier_ch = torch.tensor(sorted(ch), device=device)

    # main KV in chunks to bound temporary memory
    kv = torch.empty(rows_total, cfg.D, device=device,
                     dtype=torch.float32 if cfg.kv_dtype == "f32" else torch.bfloat16)
    step = 1 << 20
    for a in range(0, rows_total, step):
        b = min(rows_total, a + step)
        kv[a:b] = _kv_raw(cfg, b - a, g, device, outlier_ch)

    alphabet = None
    if cfg.idx_dist == "ties":
        alphabet = torch.randint(-1, 2, (64, cfg.Di), generator=g, device=device).float()
    ikeys = torch.empty(rows_total, cfg.Di, dtype=torch.uint8, device=device)
    for a in range(0, rows_total, step):
        b = min(rows_total, a + step)
        ikeys[a:b] = to_e4m3_bytes(_int_values(cfg, (b - a, cfg.Di), g, device, alphabet))

    if cfg.prefill_rows:
        R = cfg.prefill_rows
        row_seq = torch.zeros(R, dtype=torch.int32, device=device)
        row_len = torch.arange(cfg.N + 1, cfg.N + 1 + R, dtype=torch.int32, device=device)
        new_rows = torch.arange(cfg.N, cfg.N + R, dtype=torch.int64, device=device)
        swa_row_start = torch.arange(0, R, dtype=torch.int64, device=device)
        swa_rows = cfg.W - 1 + R
    else:
        R = len(lengths)
        row_seq = torch.arange(R, dtype=torch.int32, device=device)
        row_len = torch.tensor(lengths, dtype=torch.int32, device=device)
        new_rows = torch.tensor(starts + lengths - 1, dtype=torch.int64, device=device)
        swa_row_start = torch.arange(0, R, dtype=torch.int64, device=device) * cfg.W
        swa_rows = R * cfg.W
    swa_len = torch.full((R,), cfg.W, dtype=torch.int32, device=device)

    qI, w, q, swa = {}, {}, {}, {}
    for l in layers:
        if modes[l] in "FR":
            qI[l] = to_e4m3_bytes(_int_values(cfg, (R, cfg.Hi, cfg.Di), g, device))
            w[l] = _weights(cfg, (R, cfg.Hi), g, device).float()
        q[l] = torch.randn(R, cfg.H, cfg.D, generator=g, device=device).to(torch.bfloat16)
        swa[l] = to_e4m3_bytes(torch.randn(swa_rows, cfg.D, generator=g, device=device))

    return Workload(cfg=cfg, lengths=lengths,
                    seq_start=torch.tensor(starts, dtype=torch.int64, device=device),
                    rows_total=rows_total, row_seq=row_seq, row_len=row_len, kv_raw=kv,
                    ikeys=ikeys, qI=qI, w=w, q=q, swa=swa, swa_row_start=swa_row_start,
                    swa_len=swa_len, new_rows=new_rows)


# ----------------------------------------------------------------- paged layout

@dataclasses.dataclass
class PagedLayout:
    """Where a workload's packed cache rows go in a paged cache.

    Entry j of sequence s lives in cache row
    block_table[s, j // page_rows] * page_rows + j % page_rows; dst[i] is the
    cache row of packed row i.  Pages are handed out in a seeded random order,
    so neighbouring pages of a sequence are far apart in memory."""
    page_rows: int
    block_table: torch.Tensor      # [S, max_pages] int32, -1 = unmapped
    cache_rows: int
    dst: torch.Tensor              # [rows_total] int64


def paged_layout(lengths: np.ndarray, page_rows: int, seed: int, device="cpu", spare_pages: int = 0) -> PagedLayout:
    lengths = np.asarray(lengths, np.int64)
    npages = (lengths + page_rows - 1) // page_rows
    max_pages = max(int(npages.max()) if len(npages) else 1, 1)
    n_phys = int(npages.sum()) + spare_pages
    perm = np.random.Generator(np.random.PCG64(seed)).permutation(n_phys)
    bt = np.full((len(lengths), max_pages), -1, np.int64)
    dst, k = [], 0
    for s, (n, m) in enumerate(zip(lengths, npages)):
        bt[s, :m] = perm[k:k + m]
        k += int(m)
        j = np.arange(int(n))
        dst.append(bt[s, j // page_rows] * page_rows + j % page_rows)
    dst = np.concatenate(dst) if dst else np.zeros(0, np.int64)
    return PagedLayout(page_rows=page_rows, block_table=torch.tensor(bt.astype(np.int32), device=device),
                       cache_rows=n_phys * page_rows, dst=torch.tensor(dst, device=device))


def to_pages(layout: PagedLayout, packed: torch.Tensor) -> torch.Tensor:
    """Copy of packed cache rows [rows_total, ...] in the paged layout
    (unused rows zero)."""
    out = torch.zeros((layout.cache_rows,) + tuple(packed.shape[1:]), dtype=packed.dtype, device=packed.device)
    out[layout.dst] = packed
    return out


def swa_ring(swa: torch.Tensor, swa_row_start: torch.Tensor, W: int, heads: torch.Tensor) -> torch.Tensor:
    """The W window rows of each query row r stored as a ring: window row i in
    slot (heads[r] + i) mod W of the row's W slots."""
    out = swa.clone()
    i = torch.arange(W, device=swa.device)
    src = swa_row_start[:, None] + i[None, :]
    dst = swa_row_start[:, None] + (heads[:, None].long() + i[None, :]) % W
    out[dst.reshape(-1)] = swa[src.reshape(-1)]
    return out
