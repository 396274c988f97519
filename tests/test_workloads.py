"""CPU checks of the seeded input generators and page layouts that the GPU
tests and the benchmark feed to both the library and the oracle."""
import numpy as np
import torch

import workloads


def test_tiny_config_shapes_ranges_and_determinism():
    cfg = workloads.CONFIGS[1]
    a = workloads.make(cfg, "cpu")
    b = workloads.make(cfg, "cpu")
    n = cfg.N
    assert a.kv_raw.shape == (n, cfg.D) and a.ikeys.shape == (n, cfg.Di)
    assert torch.equal(a.kv_raw, b.kv_raw) and torch.equal(a.ikeys, b.ikeys)
    for l in a.qI:
        assert torch.equal(a.qI[l], b.qI[l]) and torch.equal(a.w[l], b.w[l])
    # indexer values are integers in [-3, 3], so E4M3 holds them exactly
    keys = a.ikeys.view(torch.float8_e4m3fn).float()
    assert torch.equal(keys, keys.round()) and keys.abs().max() <= 3
    # one decode row per sequence, seeing every entry; the appended entry is the last
    assert a.row_seq.tolist() == list(range(cfg.B))
    assert a.row_len.tolist() == [n] * cfg.B
    assert a.new_rows.tolist() == [n - 1]
    assert a.swa_len.tolist() == [cfg.W] * cfg.B


def test_weights_are_sixteenths_in_unit_interval():
    cfg = workloads.scaled(workloads.CONFIGS[2], B=2, N=64, w_dist="u01_16")
    wl = workloads.make(cfg, "cpu", layers=[0])
    w = wl.w[0]
    assert torch.equal(w * 16, (w * 16).round()) and w.min() >= 0 and w.max() <= 1


def test_prefill_rows_are_causal():
    cfg = workloads.scaled(workloads.CONFIGS[4], N=100, prefill_rows=7)
    wl = workloads.make(cfg, "cpu", layers=[0])
    assert wl.row_seq.tolist() == [0] * 7
    assert wl.row_len.tolist() == [101 + i for i in range(7)]
    assert wl.new_rows.tolist() == [100 + i for i in range(7)]
    # row i's window is token rows i .. i + W - 1 of one shared buffer
    assert wl.swa_row_start.tolist() == list(range(7))
    assert wl.swa[0].shape[0] == cfg.W - 1 + 7


def test_paged_layout_is_a_permutation_of_whole_pages():
    lengths = np.array([100, 0, 70, 64])
    lay = workloads.paged_layout(lengths, 16, seed=3, spare_pages=2)
    bt = lay.block_table.numpy()
    npages = (lengths + 15) // 16
    assert bt.shape == (4, npages.max())
    used = np.concatenate([bt[s, :m] for s, m in enumerate(npages)])
    assert sorted(used.tolist()) == sorted(set(used.tolist()))           # pages are not shared
    assert used.max() < lay.cache_rows // 16 and lay.cache_rows == (npages.sum() + 2) * 16
    assert all((bt[s, m:] == -1).all() for s, m in enumerate(npages))     # unused table slots
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    dst = lay.dst.numpy()
    for s, n in enumerate(lengths):
        for j in range(n):
            assert dst[starts[s] + j] == bt[s, j // 16] * 16 + j % 16
    packed = torch.arange(int(lengths.sum()) * 3).reshape(-1, 3)
    paged = workloads.to_pages(lay, packed)
    assert torch.equal(paged[lay.dst], packed)
    hole = np.setdiff1d(np.arange(lay.cache_rows), dst)
    assert (paged[torch.as_tensor(hole)] == 0).all()


def test_swa_ring_rotates_each_window():
    W, R = 5, 3
    swa = torch.arange(R * W * 2).reshape(R * W, 2)
    start = torch.arange(R) * W
    heads = torch.tensor([0, 4, 2], dtype=torch.int32)
    ring = workloads.swa_ring(swa, start, W, heads)
    for r in range(R):
        for i in range(W):
            assert torch.equal(ring[int(start[r]) + (int(heads[r]) + i) % W], swa[int(start[r]) + i])
