"""GPU parity of the multi-token (MTP) decode against the CPU oracle, through
the C ABI.  Same bars as the single-token decode: out within 2e-2 relative L2
over the whole [B,T,H,512] tensor and 5e-3 per (sequence, token, head), lse
within 1e-3 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from cases import check_parity, gpu_cache, note, oracle_cache, small_case, to_dev_bf16

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


def mtp_case(batch, tokens, heads, lens, topk, seed):
    """small_case rows and page table; T queries per sequence; token 0's list
    over the positions it sees, drafts swap 1 entry in 8, and every list also
    holds the newest positions (some of which a token may not see)."""
    case = small_case(batch, heads, lens, topk, seed=seed)
    rng = np.random.default_rng(seed + 1)
    q = wl.bf16_bits(torch.randn((batch, tokens, heads, 576),
                                 generator=torch.Generator().manual_seed(seed + 2)).to(torch.bfloat16))
    tk = np.full((batch, tokens, topk), -1, dtype=np.int32)
    for b in range(batch):
        L = int(case["lens"][b])
        base = case["topk"][b].copy()
        base[base >= L - tokens + 1] = -1
        for j in range(tokens):
            row = base.copy()
            valid = np.flatnonzero(row >= 0)
            m = valid.size // 8 if j else 0
            if m:
                row[rng.choice(valid, size=m, replace=False)] = rng.integers(0, max(L - tokens + 1 + j, 1), m)
            newest = np.arange(max(L - tokens, 0), L, dtype=np.int32)   # visible or not
            free = np.flatnonzero(row < 0)[:newest.size]
            row[free] = newest[:free.size]
            tk[b, j] = row
    case["q"] = q
    case["topk"] = tk
    return case


MTP_CASES = [
    (2, 2, 16, [3000, 900], 512),
    (3, 4, 64, [5000, 2000, 300], 2048),
    (1, 3, 16, [70000], 2048),
    (5, 2, 64, [64, 65, 129, 2, 4000], 64),
    (4, 4, 16, [2500, 2500, 90, 700], 2048),
    (2, 16, 64, [3000, 40], 1024),    # the most tokens a call takes
    (1, 16, 16, [10], 256),           # fewer positions than tokens: early tokens see none
]


@pytest.mark.parametrize("batch,tokens,heads,lens,topk", MTP_CASES,
                         ids=["B%d_T%d_H%d_K%d" % (c[0], c[1], c[2], c[4]) for c in MTP_CASES])
def test_mtp_matches_oracle(dev, smla, batch, tokens, heads, lens, topk):
    case = mtp_case(batch, tokens, heads, lens, topk, seed=batch * 7 + tokens + topk)
    note("mtp B=%d T=%d H=%d lens=%s K=%d" % (batch, tokens, heads, lens, topk))
    cache_d = gpu_cache(case, dev, smla)
    cache_o = oracle_cache(case)
    out, lse = smla.sparse_mla_decode_mtp(
        to_dev_bf16(case["q"], dev), cache_d, torch.as_tensor(case["pt"], device=dev),
        torch.as_tensor(case["lens"].astype(np.int32), device=dev),
        torch.as_tensor(case["topk"], device=dev), case["scale"])
    torch.cuda.synchronize(dev)
    ref_o, ref_l = oracle.sparse_mla_decode_mtp(case["q"], cache_o, case["pt"], case["lens"],
                                                case["topk"], case["scale"])
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    check_parity(out, ref_o, lse, ref_l)


def test_mtp_one_token_is_the_plain_decode(dev, smla):
    note("mtp T=1 vs plain decode")
    case = small_case(3, 64, [3000, 2000, 700], 2048, seed=91)
    cache_d = gpu_cache(case, dev, smla)
    args = (cache_d, torch.as_tensor(case["pt"], device=dev),
            torch.as_tensor(case["lens"].astype(np.int32), device=dev))
    q = to_dev_bf16(case["q"], dev)
    tk = torch.as_tensor(case["topk"], device=dev)
    o1, l1 = smla.sparse_mla_decode(q, *args, tk, case["scale"])
    o2, l2 = smla.sparse_mla_decode_mtp(q[:, None].contiguous(), *args, tk[:, None].contiguous(),
                                        case["scale"])
    torch.cuda.synchronize(dev)
    assert torch.equal(o1, o2[:, 0]) and torch.equal(l1, l2[:, 0])


def _sequence_mini_cache(w, b, positions, L, dev):
    """The oracle's own cache for the given logical positions of sequence b:
    every logical page holding one of them gets a page of its own, with the
    position's row quantised by the oracle from the regenerated BF16 row.
    Returns (cache [P,64,352], page table [1, ceil(L/64)])."""
    pos = np.unique(np.asarray(positions, dtype=np.int64))
    pages = np.unique(pos // 64)
    pt = np.full((1, (L + 63) // 64), -1, dtype=np.int32)
    pt[0, pages] = np.arange(pages.size, dtype=np.int32)
    cache = np.zeros((pages.size, 64, 352), dtype=np.uint8)
    rows = oracle.quant_rows(wl.bf16_bits(wl.rows_at(w, 0, b, pos, device=dev)))
    cache.reshape(-1, 352)[pt[0, pos // 64].astype(np.int64) * 64 + pos % 64] = rows
    return cache, pt


@pytest.mark.parametrize("name,tokens,sample", [("tp4", 4, [0, 31]), ("allheads", 2, [0, 63])])
def test_mtp_full_workload_sampled(dev, smla, name, tokens, sample):
    """Full-size caches and lists; a few entries of every token's list name the
    newest positions, which only later tokens see, so each token's causal
    limit decides.  The oracle gets the sequence length and computes each
    token's limit itself; sampled sequences, every token and head checked."""
    w = wl.WORKLOADS[name]
    lens = wl.context_lengths(w, 0)
    pt_np, num_pages = wl.build_page_table(w, lens, 0)
    note("mtp full %s T=%d" % (name, tokens))
    cache = torch.zeros((num_pages, 64, 352), dtype=torch.uint8, device=dev)
    wl.fill_cache(w, 0, lens, pt_np, lambda r, s: smla.kv_quant_append(r, s, cache), dev)
    tk = wl.mtp_topk(w, lens, tokens, 0)
    newest = np.arange(tokens - 1, dtype=np.int64)          # L-T+1 .. L-1: seen by later tokens
    for b in range(tk.shape[0]):
        L = int(lens[b])
        for j in range(tokens):
            tk[b, j, 1:1 + newest.size] = (L - tokens + 1 + newest).astype(np.int32)
    q = torch.cat([wl.queries(w, 0, set_id=j, device=dev)[:, None] for j in range(tokens)], 1)
    out, lse = smla.sparse_mla_decode_mtp(q.contiguous(), cache, torch.as_tensor(pt_np, device=dev),
                                          torch.as_tensor(lens.astype(np.int32), device=dev),
                                          torch.as_tensor(tk, device=dev), w.softmax_scale)
    torch.cuda.synchronize(dev)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    qbits = wl.bf16_bits(q)
    flat = cache.view(-1, 352)
    for b in sample:
        L = int(lens[b])
        sel = tk[b][tk[b] >= 0].astype(np.int64)
        mini, mpt = _sequence_mini_cache(w, b, sel, L, dev)
        # the device cache holds the same bytes at those positions
        uniq = np.unique(sel)
        slots = torch.as_tensor(pt_np[b, uniq // 64].astype(np.int64) * 64 + uniq % 64, device=dev)
        assert np.array_equal(flat[slots].cpu().numpy(),
                              mini.reshape(-1, 352)[mpt[0, uniq // 64].astype(np.int64) * 64
                                                    + uniq % 64])
        ro, rl = oracle.sparse_mla_decode_mtp(qbits[b:b + 1], mini, mpt, np.array([L]), tk[b:b + 1],
                                              w.softmax_scale)
        check_parity(out[b:b + 1], ro, lse[b:b + 1], rl, "seq %d" % b)
    del cache
    torch.cuda.empty_cache()


def test_mtp_edge_cases(dev, smla):
    """Draft tokens whose lists share only some rows, a token with no usable
    entry, rows repeated in both lists, an empty first token."""
    note("mtp edge cases")
    case = small_case(4, 16, [3000, 3000, 2000, 1500], 1024, seed=95)
    T = 2
    rng = np.random.default_rng(96)
    q = wl.bf16_bits(torch.randn((4, T, 16, 576), generator=torch.Generator().manual_seed(97))
                     .to(torch.bfloat16))
    tk = np.full((4, T, 1024), -1, dtype=np.int32)
    a = rng.choice(2999, 400, replace=False).astype(np.int32)
    # seq 0: token 1 shares only token 0's later rows
    tk[0, 0, :400] = a
    tk[0, 1, :300] = a[100:]
    # seq 1: token 1 selects nothing usable (beyond its length or -1)
    tk[1, 0, :400] = a
    tk[1, 1, :5] = [3000, 3001, -1, -7, 10 ** 6]
    # seq 2: repeated rows: token 0 twice, token 1 three times, plus others
    r = np.arange(0, 1990, 10, dtype=np.int32)
    tk[2, 0, :199] = r
    tk[2, 0, 199:201] = [5, 5]
    tk[2, 1, :199] = r[::-1]
    tk[2, 1, 199:202] = [5, 5, 5]
    tk[2, 1, 202:300] = rng.integers(0, 1999, 98)
    # seq 3: token 0 empty, token 1 sees the newest position too
    tk[3, 1, :700] = rng.choice(1500, 700, replace=False)
    tk[3, 1, 700] = 1499
    case["q"], case["topk"] = q, tk
    cache_d = gpu_cache(case, dev, smla)
    cache_o = oracle_cache(case)
    out, lse = smla.sparse_mla_decode_mtp(
        to_dev_bf16(q, dev), cache_d, torch.as_tensor(case["pt"], device=dev),
        torch.as_tensor(case["lens"].astype(np.int32), device=dev), torch.as_tensor(tk, device=dev),
        case["scale"])
    torch.cuda.synchronize(dev)
    ref_o, ref_l = oracle.sparse_mla_decode_mtp(q, cache_o, case["pt"], case["lens"], tk, case["scale"])
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all()
    assert np.isneginf(lse[1, 1]).all() and not out[1, 1].any()
    assert np.isneginf(lse[3, 0]).all() and not out[3, 0].any()
    check_parity(out, ref_o, lse, ref_l)
