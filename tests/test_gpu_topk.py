"""GPU parity of the top-k select against the CPU oracle, through the C ABI.

Several lists are correct when scores tie at the threshold, and the list's
order is unspecified, so the check compares what is unique -- the multiset
of selected scores (the top min(K, L) values) and the -1 padding -- and
checks that the rest is valid: distinct positions inside [0, L).  Where no
scores tie the selected positions must equal the oracle's as a set.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from cases import check_parity, note, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def check_lists(got: np.ndarray, scores: np.ndarray, lens: np.ndarray, K: int, exact_sets: bool):
    want = oracle.topk_select(scores, lens, K)
    for b in range(got.shape[0]):
        L = int(min(max(int(lens[b]), 0), scores.shape[1]))
        n = min(K, L)
        g, w = got[b], want[b]
        assert (g[n:] == -1).all(), b
        sel = g[:n]
        assert len(np.unique(sel)) == n, b
        assert ((sel >= 0) & (sel < L)).all(), b
        assert np.array_equal(np.sort(scores[b, sel]), np.sort(scores[b, w[:n]])), b
        if exact_sets:
            assert np.array_equal(np.sort(sel), np.sort(w[:n])), b


def run(smla, dev, scores: np.ndarray, lens: np.ndarray, K: int):
    s = torch.as_tensor(scores, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    out = smla.topk_select(s, sl, K)
    torch.cuda.synchronize(dev)
    return out.cpu().numpy()


@pytest.mark.parametrize("ld", [20000, 100000, 300000])  # workgroups of 2048, 4096, 16384 scores
def test_select_random_rows_and_lengths(dev, smla, ld):
    note("topk random rows ld=%d" % ld)
    rng = np.random.default_rng(1)
    lens = np.array([ld, 2049, 2048, 2047, 1, 0, 4097, ld - 1, 13, 8192], dtype=np.int64)
    x = rng.standard_normal((lens.size, ld)).astype(np.float32)
    got = run(smla, dev, x, lens, 2048)
    check_lists(got, x, lens, 2048, exact_sets=True)


@pytest.mark.parametrize("group", [1, 2, 63, 64, 65, 200])
def test_select_threshold_group_sizes(dev, smla, group):
    """The keys that share the threshold's first two radix digits (the top
    22 bits of the key) number `group`: up to 64 of them one wave ranks, more
    take a digit-2 histogram.  They are distinct floats 1 + 5k ulp (one
    digit-1 bin of the digit-0 bin of 1.0); 40 larger scores sit above them
    and the threshold falls inside the group."""
    note("topk threshold group of %d keys" % group)
    rng = np.random.default_rng(10 + group)
    L, K = 4096, 40 + max(1, group - 3)
    x = -1000.0 - rng.random(L).astype(np.float32) * 100  # far below
    x[:40] = 100.0 + np.arange(40, dtype=np.float32)
    bits = (0x3F800000 + 5 * np.arange(group)).astype(np.uint32)
    x[40:40 + group] = bits.view(np.float32)
    x = x[rng.permutation(L)].astype(np.float32)
    rows = np.stack([x, np.roll(x, 7)])
    lens = np.array([L, L - 1], dtype=np.int64)
    got = run(smla, dev, rows, lens, K)
    check_lists(got, rows, lens, K, exact_sets=True)


@pytest.mark.parametrize("K", [1, 17, 256, 2048])
def test_select_ties_at_the_threshold(dev, smla, K):
    note("topk ties K=%d" % K)
    rng = np.random.default_rng(2 + K)
    ld = 12000
    lens = np.array([12000, 9000, 5000, 3000], dtype=np.int64)
    x = rng.integers(-20, 21, size=(4, ld)).astype(np.float32)    # 41 distinct values
    x[3] = 7.0                                                      # one row all equal
    x[2, ::2] = -0.0
    x[2, 1::2] = 0.0                                                # signed zeros
    got = run(smla, dev, x, lens, K)
    check_lists(got, x, lens, K, exact_sets=False)


def test_select_extreme_values_and_signs(dev, smla):
    note("topk extreme values")
    rng = np.random.default_rng(3)
    ld = 8192
    x = (rng.standard_normal((3, ld)) * 1e30).astype(np.float32)
    x[1] = -np.abs(rng.standard_normal(ld)).astype(np.float32)     # all negative
    x[2] = rng.standard_normal(ld).astype(np.float32) * 1e-40      # subnormals
    lens = np.array([ld, ld, ld])
    got = run(smla, dev, x, lens, 500)
    check_lists(got, x, lens, 500, exact_sets=False)


def test_select_workspace_reuse_across_shapes(dev, smla):
    """The workspace is left ready: calls of different shapes in a row on the
    same workspace all give valid lists."""
    note("topk workspace reuse")
    rng = np.random.default_rng(4)
    ws = torch.zeros(int(smla.lib.smla_topk_workspace_bytes(16, 70000)), dtype=torch.uint8,
                     device=dev)
    for trial, (B, ld, K) in enumerate([(16, 30000, 2048), (3, 5000, 64), (16, 30000, 2048),
                                        (9, 70000, 1000), (1, 4, 2)]):
        x = rng.standard_normal((B, ld)).astype(np.float32)
        lens = rng.integers(0, ld + 1, size=B)
        lens[0] = ld
        out = smla.topk_select(torch.as_tensor(x, device=dev),
                               torch.as_tensor(lens.astype(np.int32), device=dev), K, workspace=ws)
        torch.cuda.synchronize(dev)
        check_lists(out.cpu().numpy(), x, lens, K, exact_sets=True)
        assert not ws.any(), "the select leaves its workspace all zero"


def test_select_overflowing_candidates(dev, smla):
    """More keys in the threshold's first-digit bin than the candidate buffer
    holds (16384): the finish reads them from the scores."""
    note("topk candidate overflow")
    rng = np.random.default_rng(5)
    ld = 40000
    x = np.full((3, ld), 1.0, dtype=np.float32)               # all in one bin
    x[1] = 1.0 + rng.integers(0, 64, ld).astype(np.float32) / 1024.0   # one bin, 64 values
    x[2] = rng.standard_normal(ld).astype(np.float32)
    lens = np.array([ld, ld - 3, ld])
    got = run(smla, dev, x, lens, 2048)
    check_lists(got, x, lens, 2048, exact_sets=False)


@pytest.mark.parametrize("name", ["allheads", "million", "ragged"])
def test_select_full_workloads(dev, smla, name):
    w = wl.WORKLOADS[name]
    lens = wl.context_lengths(w, 0)
    note("topk full %s" % name)
    scores = wl.index_scores(w, lens, 0, device=dev)
    out = smla.topk_select(scores, torch.as_tensor(lens.astype(np.int32), device=dev), w.topk)
    torch.cuda.synchronize(dev)
    x = scores.cpu().numpy()
    check_lists(out.cpu().numpy(), x, lens, w.topk, exact_sets=True)


def test_select_then_decode(dev, smla):
    """The selected list feeds the decode: the result equals the oracle's
    decode over the oracle's list (same set, other order)."""
    note("topk -> decode")
    from cases import gpu_cache, oracle_cache, small_case
    case = small_case(3, 64, [5000, 3000, 900], 2048, seed=81)
    ld = 5000
    rng = np.random.default_rng(82)
    x = rng.standard_normal((3, ld)).astype(np.float32)
    lens = case["lens"]
    tk = smla.topk_select(torch.as_tensor(x, device=dev),
                          torch.as_tensor(lens.astype(np.int32), device=dev), 2048)
    cache_d = gpu_cache(case, dev, smla)
    q = to_dev_bf16(case["q"], dev)
    out, lse = smla.sparse_mla_decode(q, cache_d, torch.as_tensor(case["pt"], device=dev),
                                      torch.as_tensor(lens.astype(np.int32), device=dev), tk,
                                      case["scale"])
    torch.cuda.synchronize(dev)
    ref_tk = oracle.topk_select(x, lens, 2048)
    ref_o, ref_l = oracle.sparse_mla_decode(case["q"], oracle_cache(case), case["pt"], lens,
                                            ref_tk, case["scale"])
    check_parity(out.cpu().numpy(), ref_o, lse.cpu().numpy(), ref_l)
