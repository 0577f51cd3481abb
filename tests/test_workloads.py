"""CPU checks of the seeded input generators (shapes, structure, determinism)."""
import numpy as np
import torch

import workloads as wl


def test_page_tables_are_permutations():
    for name in ("tiny", "tp4", "ragged"):
        w = wl.WORKLOADS[name]
        lens = wl.context_lengths(w, 0)
        pt, npages = wl.build_page_table(w, lens, 0)
        used = np.concatenate([pt[b, :(int(L) + 63) // 64] for b, L in enumerate(lens)])
        assert np.array_equal(np.sort(used), np.arange(npages))
        if name == "tiny":
            assert np.array_equal(pt[0], np.arange(64))


def test_topk_lists():
    w = wl.WORKLOADS["ragged"]
    lens = wl.context_lengths(w, 0)
    assert lens.min() >= 1024 and lens.max() <= 146000
    tk = wl.topk_indices(w, lens, 0)
    for b, L in enumerate(lens):
        v = tk[b][tk[b] >= 0]
        assert v.size == min(2048, L) and np.unique(v).size == v.size and v.max() < L
        assert (tk[b][v.size:] == -1).all()
    w3 = wl.WORKLOADS["allheads"]
    l3 = np.array([140000, 140000])
    t3 = wl.topk_indices(w3, l3, 0)
    for b in range(2):
        assert np.unique(t3[b]).size == 2048
        assert ((t3[b] >= 140000 - 6000).sum()) == 1024
        assert not np.all(np.diff(t3[b]) > 0)           # shuffled, not sorted
    assert not np.array_equal(wl.topk_indices(w3, l3, 0, set_id=1), t3)


def test_rows_are_reproducible_by_position():
    w = wl.WORKLOADS["allheads"]
    a = wl.kv_rows(w, 0, 3, 8000, 500)
    b = wl.rows_at(w, 0, 3, np.arange(8000, 8500)[::-1])
    assert torch.equal(a, b.flip(0))
    ch = wl.outlier_channels(w, 0)
    assert ch.size == 8
    x = wl.kv_chunk(w, 0, 0, 0).float()
    big = x[:, ch].abs().mean() / x.abs().mean()
    assert big > 6                                   # outlier channels scaled x8
