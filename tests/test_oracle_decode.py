"""CPU pins of the oracle's sparse MLA decode.

The decode oracle is fixed against: dense attention computed by a library
routine (torch's scaled_dot_product_attention and logsumexp, fp64) over rows
decoded independently of the oracle; closed forms (one-hot, uniform,
single entry, empty selection); and invariances (padding, out-of-range
entries, page relocation, list order).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl
from test_oracle_format import _independent_decode, bf16_bits_to_f64, _f64_to_bf16_exact

SCALE = 1.0 / math.sqrt(576)


def make_case(B=2, H=4, lens=(200, 130), K=None, seed=0, pages="shuffled", extra_pages=3):
    """Small random cache: returns dict with q bits, cache, page table, lens, bf16 rows."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    npg = [(int(L) + 63) // 64 for L in lens]
    total = sum(npg) + extra_pages
    perm = rng.permutation(total).astype(np.int32) if pages != "identity" else \
        np.arange(total, dtype=np.int32)
    maxp = max(npg)
    pt = np.full((B, maxp), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        pt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    cache = np.zeros((total, 64, 352), dtype=np.uint8)
    rows = []
    for b in range(B):
        x = torch.randn((int(lens[b]), 576), generator=torch.Generator().manual_seed(seed * 100 + b))
        x[:, :8] *= 8
        bits = wl.bf16_bits(x.to(torch.bfloat16))
        slots = wl.slots_for(pt, b, 0, int(lens[b]))
        assert oracle.kv_quant_append(bits, slots, cache) == lens[b]
        rows.append(bits)
    q = wl.bf16_bits(torch.randn((B, H, 576), generator=torch.Generator().manual_seed(seed + 7))
                     .to(torch.bfloat16))
    return dict(q=q, cache=cache, pt=pt, lens=lens, rows=rows)


def decoded_logical(case, b):
    """Row values of sequence b in token order, decoded without the oracle."""
    L = int(case["lens"][b])
    slots = wl.slots_for(case["pt"], b, 0, L).astype(np.int64)
    raw = case["cache"].reshape(-1, 352)[slots]
    return _independent_decode(raw)


def library_attention(q_bits, Kmat, scale):
    """Dense softmax attention by torch's SDPA in fp64; V = first 512 columns."""
    q = torch.from_numpy(bf16_bits_to_f64(q_bits))                  # [H,576]
    Kt = torch.from_numpy(Kmat)                                       # [n,576]
    H, n = q.shape[0], Kt.shape[0]
    k4 = Kt[None, None].expand(1, H, n, 576).contiguous()
    v4 = Kt[None, None, :, :512].expand(1, H, n, 512).contiguous()
    out = F.scaled_dot_product_attention(q[None, :, None, :], k4, v4, scale=scale)
    lse = torch.logsumexp(scale * (q @ Kt.T), dim=-1)
    return out[0, :, 0, :].numpy(), lse.numpy()


def run(case, topk, scale=SCALE, lens=None, pt=None, cache=None):
    return oracle.sparse_mla_decode(case["q"], case["cache"] if cache is None else cache,
                                    case["pt"] if pt is None else pt,
                                    case["lens"] if lens is None else lens, topk, scale)


def test_full_topk_reduces_to_dense_attention():
    case = make_case(B=2, H=5, lens=(200, 129), seed=1)
    K = 200
    rng = np.random.default_rng(2)
    topk = np.full((2, K), -1, dtype=np.int32)
    topk[0] = rng.permutation(200)
    topk[1, :129] = rng.permutation(129)
    out, lse = run(case, topk)
    for b in range(2):
        ref_o, ref_l = library_attention(case["q"][b], decoded_logical(case, b), SCALE)
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-13, atol=1e-13)


def test_sparse_selection_is_attention_over_selected_rows():
    case = make_case(B=2, H=3, lens=(300, 77), seed=3)
    rng = np.random.default_rng(4)
    K = 64
    topk = np.full((2, K), -1, dtype=np.int32)
    topk[0] = rng.choice(300, K, replace=False)
    topk[1, :40] = rng.choice(77, 40, replace=False)
    out, lse = run(case, topk)
    for b in range(2):
        sel = topk[b][topk[b] >= 0]
        ref_o, ref_l = library_attention(case["q"][b], decoded_logical(case, b)[sel], SCALE)
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-13, atol=1e-13)


def test_one_hot_softmax():
    case = make_case(B=1, H=2, lens=(128,), seed=5)
    Kd = decoded_logical(case, 0)
    t_star = int(np.argmax((Kd ** 2).sum(1)))
    k = Kd[t_star]
    # q = 2^j * k (exact in bf16); pick j so the winning score leads by >= 40
    others = np.delete(Kd, t_star, axis=0)
    gap = SCALE * (k @ k - (others @ k).max())
    j = int(math.ceil(math.log2(40.0 / gap)))
    q = _f64_to_bf16_exact(np.ldexp(k, j))
    qq = np.stack([q, q])[None]
    case["q"] = qq
    topk = np.arange(128, dtype=np.int32)[None]
    out, lse = run(case, topk)
    s_star = SCALE * float(bf16_bits_to_f64(q) @ k)
    for h in range(2):
        np.testing.assert_allclose(out[0, h], k[:512], rtol=0, atol=1e-12 * np.abs(k).max())
        assert abs(lse[0, h] - s_star) < 1e-12 * abs(s_star)


def test_uniform_scores_give_mean_and_log_count():
    case = make_case(B=1, H=3, lens=(150,), seed=6)
    Kd = decoded_logical(case, 0)
    sel = np.array([5, 77, 149, 5, 0, 64, 63], dtype=np.int32)     # 5 appears twice
    topk = np.concatenate([sel, np.full(9, -1, np.int32)])[None]
    out, lse = run(case, topk, scale=0.0)
    want = Kd[sel, :512].mean(axis=0)
    for h in range(3):
        np.testing.assert_allclose(out[0, h], want, rtol=1e-14, atol=1e-14)
        assert lse[0, h] == pytest.approx(math.log(len(sel)), abs=1e-15)


def test_single_entry_is_exact():
    case = make_case(B=1, H=4, lens=(100,), seed=7)
    Kd = decoded_logical(case, 0)
    topk = np.full((1, 32), -1, dtype=np.int32)
    topk[0, 17] = 42
    out, lse = run(case, topk)
    q = bf16_bits_to_f64(case["q"][0])
    for h in range(4):
        assert np.array_equal(out[0, h], Kd[42, :512])           # w = l = 1
        assert lse[0, h] == pytest.approx(SCALE * (q[h] @ Kd[42]), rel=1e-14, abs=1e-15)


def test_empty_selection():
    case = make_case(B=2, H=2, lens=(100, 0 + 64), seed=8)
    topk = np.full((2, 8), -1, dtype=np.int32)
    topk[1] = [64, 65, 1000, -5, 70, 99, 127, 64]     # all >= L_1 = 64 or negative
    out, lse = run(case, topk)
    assert not out.any()
    assert np.isneginf(lse).all()


def test_padding_and_out_of_range_entries_change_nothing():
    case = make_case(B=2, H=3, lens=(260, 70), seed=9)
    rng = np.random.default_rng(10)
    base = np.stack([rng.choice(260, 50, replace=False),
                     np.concatenate([rng.choice(70, 30, replace=False), np.full(20, -1)])])
    base = base.astype(np.int32)
    base[0, :2] = [257, 259]                         # rows of page 4, used below
    o1, l1 = run(case, base)
    junk = np.array([-1, -7, 260, 10 ** 6, -2 ** 31], dtype=np.int32)
    padded = np.full((2, 50 + 2 * junk.size), -1, dtype=np.int32)
    for b in range(2):
        v = base[b]
        mixed = list(v[:20]) + list(junk) + list(v[20:]) + list(junk)
        padded[b, :len(mixed)] = mixed
    padded[1][padded[1] == 260] = 70                               # t == L_1 is out of range
    o2, l2 = run(case, padded)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # an entry whose page id is outside the cache is skipped as well
    pt = case["pt"].copy()
    pt[0, 4] = case["cache"].shape[0] + 5                           # tokens 256..259
    o3, l3 = run(case, base, pt=pt)
    keep = np.where((base[0] >= 256) & (base[0] < 260), -1, base[0])
    o4, l4 = run(case, np.stack([keep, base[1]]).astype(np.int32), pt=pt)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_page_relocation_changes_nothing():
    case = make_case(B=2, H=2, lens=(300, 200), seed=11, extra_pages=4)
    rng = np.random.default_rng(12)
    topk = np.stack([rng.choice(300, 100, replace=False),
                     rng.choice(200, 100, replace=False)]).astype(np.int32)
    o1, l1 = run(case, topk)
    P = case["cache"].shape[0]
    move = rng.permutation(P)                          # physical page p -> move[p]
    cache2 = np.zeros_like(case["cache"])
    cache2[move] = case["cache"]
    pt2 = np.where(case["pt"] >= 0, move[np.maximum(case["pt"], 0)], -1).astype(np.int32)
    o2, l2 = run(case, topk, pt=pt2, cache=cache2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_list_order_only_changes_rounding():
    case = make_case(B=1, H=3, lens=(400,), seed=13)
    rng = np.random.default_rng(14)
    topk = rng.choice(400, 256, replace=False).astype(np.int32)[None]
    o1, l1 = run(case, topk)
    o2, l2 = run(case, topk[:, rng.permutation(256)])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14, atol=1e-14)


def test_lse_normalises_the_weights():
    case = make_case(B=1, H=4, lens=(256,), seed=15)
    Kd = decoded_logical(case, 0)
    topk = np.arange(0, 256, 3, dtype=np.int32)[None]
    _, lse = run(case, topk)
    q = bf16_bits_to_f64(case["q"][0])
    s = SCALE * (q @ Kd[topk[0]].T)                                 # [H, n]
    tot = np.exp(s - lse[0][:, None]).sum(axis=1)
    np.testing.assert_allclose(tot, 1.0, rtol=0, atol=1e-13)


def test_oracle_on_generated_tiny_workload():
    """The generators' tiny workload runs through the oracle end to end."""
    w = wl.WORKLOADS["tiny"]
    lens = wl.context_lengths(w, 0)
    pt, npages = wl.build_page_table(w, lens, 0)
    cache = np.zeros((npages, 64, 352), dtype=np.uint8)
    for b, t0, rows, slots in wl.iter_fill(w, 0, lens, pt):
        oracle.kv_quant_append(wl.bf16_bits(rows), slots, cache)
    topk = wl.topk_indices(w, lens, 0)
    q = wl.bf16_bits(wl.queries(w, 0))
    out, lse = oracle.sparse_mla_decode(q, cache, pt, lens, topk, w.softmax_scale)
    assert out.shape == (1, 16, 512) and np.isfinite(out).all() and np.isfinite(lse).all()
    Kd = _independent_decode(cache.reshape(-1, 352)[topk[0].astype(np.int64)])
    ref_o, ref_l = library_attention(q[0], Kd, w.softmax_scale)
    np.testing.assert_allclose(out[0], ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse[0], ref_l, rtol=1e-13, atol=1e-13)


def test_entries_past_the_page_table_are_skipped():
    """A context longer than its page-table row (seq_lens > max_pages * 64):
    an entry t with t / 64 >= max_pages has no page and is skipped, so the
    result is attention over the selected rows the table does hold, computed
    by the library routine over rows decoded without the oracle."""
    case = make_case(B=2, H=3, lens=(300, 260), seed=17)
    rng = np.random.default_rng(18)
    topk = np.stack([rng.choice(300, 120, replace=False),
                     rng.choice(260, 120, replace=False)]).astype(np.int32)
    max_pages = 3                                    # tokens 0..191 have a page
    narrow = np.ascontiguousarray(case["pt"][:, :max_pages])
    assert (topk >= 64 * max_pages).sum(axis=1).min() > 20
    out, lse = run(case, topk, pt=narrow)
    for b in range(2):
        sel = topk[b][topk[b] < 64 * max_pages]
        ref_o, ref_l = library_attention(case["q"][b], decoded_logical(case, b)[sel], SCALE)
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-13, atol=1e-13)
    # only such entries: nothing usable
    only_past = np.where(topk >= 64 * max_pages, topk, -1).astype(np.int32)
    out2, lse2 = run(case, only_past, pt=narrow)
    assert not out2.any() and np.isneginf(lse2).all()
