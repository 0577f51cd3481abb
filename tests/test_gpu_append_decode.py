"""GPU parity of the fused append-and-decode entry point, through the C ABI.

smla_append_decode stands for smla_kv_quant_append of each sequence's newest
row followed by smla_sparse_mla_decode.  The same inputs go through both
routes on two copies of one cache: the cache bytes, out and lse must be
bit-identical (the fused kernel quantises the row with the append's own code
and decodes with the same arithmetic), and both must match the oracle's
append-then-decode within the parity bars.  The lists take the new token 0,
1 or several times, and one sequence's new row is skipped (slot -1)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from cases import check_parity, note, small_case, to_dev_bf16

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


CASES = [
    # batch, heads, lens, topk, copies of the new token per list (by sequence)
    (4, 16, [3000, 5000, 700, 2049], 512, [0, 1, 3, 1]),
    (3, 64, [9000, 2500, 5000], 2048, [1, 2, 0]),
    (5, 64, [4100, 130, 2300, 64, 7000], 256, [1, 1, 1, 1, 0]),
    (40, 16, [1500 + 97 * i for i in range(40)], 1024, [i % 3 for i in range(40)]),
]


def fused_against_two_calls(dev, smla, c, new_slots):
    """The newest token of every sequence appended at new_slots (-1: not
    appended) and decoded, by the fused call and by the two calls, on copies
    of one cache holding every older token; then both against the oracle."""
    B = c["q"].shape[0]
    lens = c["lens"]
    new_bits = np.stack([c["rows"][b][int(lens[b]) - 1] for b in range(B)])
    base = torch.zeros((c["num_pages"], 64, 352), dtype=torch.uint8, device=dev)
    for b in range(B):
        n = int(lens[b]) - 1
        if n:
            smla.kv_quant_append(to_dev_bf16(c["rows"][b][:n], dev),
                                 torch.as_tensor(wl.slots_for(c["pt"], b, 0, n), device=dev), base)
    q = to_dev_bf16(c["q"], dev)
    pt = torch.as_tensor(np.ascontiguousarray(c["pt"]), device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    tk = torch.as_tensor(np.ascontiguousarray(c["topk"]), device=dev)
    rows_d = to_dev_bf16(new_bits, dev)
    slots_d = torch.as_tensor(new_slots, device=dev)

    cache_two = base.clone()
    smla.kv_quant_append(rows_d, slots_d, cache_two)
    o2, l2 = smla.sparse_mla_decode(q, cache_two, pt, sl, tk, c["scale"])
    cache_one = base.clone()
    o1, l1 = smla.append_decode(rows_d, slots_d, q, cache_one, pt, sl, tk, c["scale"])
    torch.cuda.synchronize(dev)
    assert torch.equal(cache_one, cache_two), "cache bytes differ from the two-call route"
    assert torch.equal(o1, o2), "out differs from the two-call route"
    assert torch.equal(l1, l2), "lse differs from the two-call route"

    # the oracle's append, then its decode
    ref_cache = np.zeros((c["num_pages"], 64, 352), dtype=np.uint8)
    for b in range(B):
        n = int(lens[b]) - (0 if new_slots[b] >= 0 else 1)
        if n:
            oracle.kv_quant_append(c["rows"][b][:n], wl.slots_for(c["pt"], b, 0, n), ref_cache)
    assert np.array_equal(cache_one.cpu().numpy(), ref_cache)
    ro, rl = oracle.sparse_mla_decode(c["q"], ref_cache, c["pt"], lens, c["topk"], c["scale"])
    check_parity(o1.cpu().numpy(), ro, l1.cpu().numpy(), rl, "append_decode")
    return o1.cpu().numpy(), l1.cpu().numpy()


def newest_slots(c):
    lens = c["lens"]
    return np.array([wl.slots_for(c["pt"], b, int(lens[b]) - 1, 1)[0] for b in range(lens.size)],
                    dtype=np.int32)


@pytest.mark.parametrize("case_i", range(len(CASES)))
def test_append_decode_matches_two_calls(dev, smla, case_i):
    B, H, lens, K, copies = CASES[case_i]
    note("append_decode B=%d H=%d K=%d" % (B, H, K))
    c = small_case(B, H, lens, K, seed=40 + case_i, pad=K // 8)
    rng = np.random.default_rng(70 + case_i)
    lens = c["lens"]
    # the newest token's position in some lists (replacing entries)
    for b in range(B):
        if copies[b]:
            pos = rng.choice(K, copies[b], replace=False)
            c["topk"][b, pos] = int(lens[b]) - 1
    new_slots = newest_slots(c)
    new_slots[-1] = -1  # the last sequence's row is not appended
    fused_against_two_calls(dev, smla, c, new_slots)


def test_append_decode_first_tokens_and_empty_lists(dev, smla):
    """Edge cases: a sequence whose only token is the new one (its list
    selects that token alone), a list with no usable entry (out 0, lse -inf,
    and the new row still reaches the cache), a new token that opens a page
    (position 64) and is the last entry of its list, and one in the middle
    of a 64-head list."""
    note("append_decode edge cases")
    K = 256
    c = small_case(4, 64, [1, 40, 65, 700], K, seed=77)
    c["topk"][0, :] = -1
    c["topk"][0, 5] = 0
    c["topk"][1, :] = -1
    c["topk"][2, :] = -1
    c["topk"][2, :65] = np.arange(65, dtype=np.int32)
    c["topk"][3, K // 2] = 699
    out, lse = fused_against_two_calls(dev, smla, c, newest_slots(c))
    assert not out[1].any() and np.isneginf(lse[1]).all()


def test_append_decode_full_tp4_step(dev, smla):
    """One decode step at the TP4-share shape (32 sequences, 16 heads, 32K
    contexts, top-k 2048), the newest token in every list: fused against the
    two calls, bit for bit."""
    w = wl.WORKLOADS["tp4"]
    note("append_decode full tp4")
    lens = wl.context_lengths(w, 0)
    pt_np, num_pages = wl.build_page_table(w, lens, 0)
    cache = torch.zeros((num_pages, 64, 352), dtype=torch.uint8, device=dev)
    wl.fill_cache(w, 0, lens, pt_np, lambda r, s: smla.kv_quant_append(r, s, cache), dev,
                  tail=1)
    rows, slots = wl.tail_rows(w, 0, lens, pt_np, dev, 1)
    tk = wl.topk_indices(w, lens, 0)
    tk[:, 0] = (lens - 1).astype(np.int32)
    q = wl.queries(w, 0, device=dev)
    pt = torch.as_tensor(pt_np, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    tk_d = torch.as_tensor(tk, device=dev)
    cache_two = cache.clone()
    smla.kv_quant_append(rows, slots, cache_two)
    o2, l2 = smla.sparse_mla_decode(q, cache_two, pt, sl, tk_d, w.softmax_scale)
    o1, l1 = smla.append_decode(rows, slots, q, cache, pt, sl, tk_d, w.softmax_scale)
    torch.cuda.synchronize(dev)
    assert torch.equal(cache, cache_two)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_append_decode_rejects_bad_arguments(dev, smla):
    c = small_case(2, 16, [300, 200], 64, seed=3)
    cache = torch.zeros((c["num_pages"], 64, 352), dtype=torch.uint8, device=dev)
    q = to_dev_bf16(c["q"], dev)
    pt = torch.as_tensor(np.ascontiguousarray(c["pt"]), device=dev)
    sl = torch.as_tensor(c["lens"].astype(np.int32), device=dev)
    tk = torch.as_tensor(np.ascontiguousarray(c["topk"]), device=dev)
    rows = torch.zeros((2, 576), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        smla.append_decode(rows[:1], torch.zeros(2, dtype=torch.int32, device=dev), q, cache, pt, sl,
                           tk, c["scale"])
    with pytest.raises(ValueError):
        smla.append_decode(rows, torch.zeros(3, dtype=torch.int32, device=dev), q, cache, pt, sl,
                           tk, c["scale"])
