"""GPU parity of the HIP path against the CPU oracle (through the C ABI).

Bars: cache bytes bit-exact; decode out within 2e-2 relative L2 over the
whole [B,H,512] tensor and within 5e-3 for every (b,h) row, lse within 1e-3
absolute (max over (b,h)).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from cases import (HEAD_TOL, decode_plan, LSE_TOL, OUT_TOL, check_parity, gpu_cache, gpu_decode, lse_err, note,
                   oracle_cache, oracle_decode, rel_l2, small_case, to_dev_bf16)

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


def _append_and_read(smla, dev, bits: np.ndarray) -> np.ndarray:
    n = bits.shape[0]
    pages = (n + 63) // 64
    cache = torch.zeros((pages, 64, 352), dtype=torch.uint8, device=dev)
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    smla.kv_quant_append(to_dev_bf16(bits, dev), slots, cache)
    torch.cuda.synchronize(dev)
    return cache.view(-1, 352)[:n].cpu().numpy()


# --------------------------------------------------------------------------
# kv_quant_append: bit-exact
# --------------------------------------------------------------------------

def test_quant_random_rows_bit_exact(dev, smla):
    note("quant random rows n=5000")
    g = torch.Generator().manual_seed(1)
    x = torch.randn((5000, 576), generator=g)
    x[:1000] *= 8
    x[1000:2000] *= 1e-3
    x[2000:2500] *= 300.0
    x[2500:2600, 100:300] = 0
    bits = wl.bf16_bits(x.to(torch.bfloat16))
    bits[2600:2610, :64] = 0x8000                       # -0 blocks
    got = _append_and_read(smla, dev, bits)
    want = oracle.quant_rows(bits)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


def test_quant_every_amax_bit_exact(dev, smla):
    """Every positive finite BF16 value as a block maximum, the other 15 values
    of the block drawn at or below it; covers every scale decision."""
    note("quant every bf16 amax")
    bits_all = np.arange(0x0001, 0x7F80, dtype=np.uint32).astype(np.uint16)   # positive finite
    nblk = bits_all.size
    rows = (nblk + 31) // 32
    rng = np.random.default_rng(2)
    x = np.zeros((rows * 32, 16), dtype=np.uint16)
    amax = np.concatenate([bits_all, bits_all[:rows * 32 - nblk]])
    # values <= amax in magnitude: random bit patterns below amax (monotone in bits)
    lower = (rng.random((rows * 32, 15)) * amax[:, None].astype(np.float64)).astype(np.uint16)
    x[:, 0] = amax
    x[:, 1:] = lower
    x[:, 1:] |= (rng.integers(0, 2, size=(rows * 32, 15)) << 15).astype(np.uint16)   # signs
    for r in range(rows * 32):
        x[r] = x[r, rng.permutation(16)] if r % 5 == 0 else x[r]
    lat = x.reshape(rows, 512)
    rope = rng.integers(0, 0x7F80, size=(rows, 64)).astype(np.uint16)
    bits = np.concatenate([lat, rope], axis=1)
    got = _append_and_read(smla, dev, bits)
    want = oracle.quant_rows(bits)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


def test_quant_every_bf16_rope_and_e2m1_ties(dev, smla):
    note("quant every bf16 rope value, e2m1 ties")
    finite = np.array([b for b in range(65536) if ((b >> 7) & 0xFF) != 0xFF], dtype=np.uint16)
    nrows = (finite.size + 63) // 64
    rope = np.resize(finite, nrows * 64).reshape(nrows, 64)
    # latent: blocks whose values sit exactly on e2m1 midpoints of their own scale
    lat = np.zeros((nrows, 512), dtype=np.uint16)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0, 4.0, 2.0, 1.0,
                     1.5, 0.0, 6.0])
    scales = oracle.e4m3_value(np.arange(1, 0x7F, dtype=np.uint8))
    for r in range(nrows):
        S = scales[r % scales.size]
        vals = (mids * S).astype(np.float32)            # exact: <= 7 significant bits
        u = vals.view(np.uint32)
        assert not (u & 0xFFFF).any()
        blk = (u >> 16).astype(np.uint16)
        blk[::3] |= 0x8000
        lat[r] = np.tile(blk, 32)
    bits = np.concatenate([lat, rope], axis=1)
    got = _append_and_read(smla, dev, bits)
    want = oracle.quant_rows(bits)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


def test_quant_slot_mapping_skips_and_leaves_others(dev, smla):
    note("quant slot mapping")
    n = 300
    bits = wl.bf16_bits(torch.randn((n, 576), generator=torch.Generator().manual_seed(3))
                        .to(torch.bfloat16))
    pages = 6
    slots = np.random.default_rng(4).permutation(pages * 64)[:n].astype(np.int32)
    slots[::7] = -1
    slots[5] = pages * 64            # one past the end
    slots[6] = 2 ** 31 - 1
    cache = torch.full((pages, 64, 352), 0xAB, dtype=torch.uint8, device=dev)
    smla.kv_quant_append(to_dev_bf16(bits, dev), torch.as_tensor(slots, device=dev), cache)
    torch.cuda.synchronize(dev)
    want = np.full((pages, 64, 352), 0xAB, dtype=np.uint8)
    oracle.kv_quant_append(bits, slots, want)
    assert np.array_equal(cache.cpu().numpy(), want)


# --------------------------------------------------------------------------
# sparse_mla_decode: small problems, several tiles, ragged tails
# --------------------------------------------------------------------------

DECODE_CASES = [
    # (batch, heads, lens, topk, extra kwargs)
    (1, 16, [4096], 256, {}),
    (3, 16, [3000, 777, 64], 512, {}),
    (2, 64, [5000, 1500], 2048, {}),
    (5, 64, [2100, 300, 64, 1, 4000], 2048, {}),
    (4, 16, [2500, 2500, 90, 700], 2048, dict(pad=1500)),
    (2, 16, [1000, 1000], 100, dict(dup=10, junk=5)),
    (2, 64, [333, 129], 17, dict(junk=3)),
    (1, 64, [70000], 2048, {}),
    (6, 16, [64, 65, 127, 128, 129, 1], 64, {}),
    # split counts that are not a power of two (11 and 7): the merge's
    # padded split slots carry weight 0
    (12, 64, [4100, 2049, 3000, 150, 5000, 2048, 64, 999, 4444, 2500, 1, 3333], 2048, {}),
    (40, 16, [1200 + 97 * i for i in range(40)], 1024, dict(pad=300)),
]


@pytest.mark.parametrize("batch,heads,lens,topk,kw", DECODE_CASES,
                         ids=["B%d_H%d_K%d_%d" % (c[0], c[1], c[3], i)
                              for i, c in enumerate(DECODE_CASES)])
def test_decode_matches_oracle(dev, smla, batch, heads, lens, topk, kw):
    case = small_case(batch, heads, lens, topk, seed=batch * 100 + topk, **kw)
    note("decode B=%d H=%d lens=%s K=%d %s" % (batch, heads, lens, topk, kw))
    cache_d = gpu_cache(case, dev, smla)
    cache_o = oracle_cache(case)
    assert np.array_equal(cache_d.cpu().numpy(), cache_o)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)


def test_decode_empty_selections(dev, smla):
    note("decode empty selections")
    case = small_case(3, 64, [100, 50, 10], 64, seed=5)
    case["topk"][:] = -1
    case["topk"][1, :5] = [50, 51, 99, -3, 10 ** 6]     # all out of range for L=50
    cache_d = gpu_cache(case, dev, smla)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    assert not out.any()
    assert np.isneginf(lse).all()
    # a page id outside the cache is skipped too
    case2 = small_case(1, 16, [128], 64, seed=6)
    case2["pt"][0, 1] = case2["num_pages"] + 3          # tokens 64..127
    case2["topk"][0] = np.arange(64, 128)
    out2, lse2 = gpu_decode(case2, gpu_cache(small_case(1, 16, [128], 64, seed=6), dev, smla),
                            dev, smla)
    assert not out2.any() and np.isneginf(lse2).all()


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_decode_page_table_narrower_than_context(dev, smla, fmt):
    """seq_lens past max_pages * 64: entries whose page-table column does not
    exist are skipped (no load), as the oracle skips them."""
    note("decode with a page table narrower than the context (%s)" % fmt)
    case = small_case(3, 64, [3000, 2500, 700], 1024, seed=71)
    cache_o = oracle_cache(case, fmt)
    cache_d = gpu_cache(case, dev, smla, fmt)
    max_pages = 20                                      # tokens 0..1279 have a page
    case["pt"] = np.ascontiguousarray(case["pt"][:, :max_pages])
    assert ((case["topk"] >= 64 * max_pages).sum(axis=1)[:2] > 300).all()
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)
    # the same rows selected with the entries past the table removed: equal
    # results (the usable entries keep their order)
    case_k = dict(case, topk=np.where(case["topk"] < 64 * max_pages, case["topk"], -1)
                  .astype(np.int32))
    out_k, lse_k = gpu_decode(case_k, cache_d, dev, smla)
    assert np.allclose(out_k, out, rtol=0, atol=1e-6) and np.array_equal(np.isneginf(lse_k),
                                                                         np.isneginf(lse))


def test_decode_deterministic(dev, smla):
    note("decode determinism")
    case = small_case(2, 64, [3000, 2000], 2048, seed=7)
    cache_d = gpu_cache(case, dev, smla)
    a = gpu_decode(case, cache_d, dev, smla)
    b = gpu_decode(case, cache_d, dev, smla)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_decode_invariances(dev, smla):
    """Page relocation is bit-identical; list permutation and -1 padding only
    move rounding."""
    note("decode invariances")
    case = small_case(2, 16, [2000, 900], 1024, seed=8, pad=200)
    cache_d = gpu_cache(case, dev, smla)
    base_o, base_l = gpu_decode(case, cache_d, dev, smla)
    # relocate pages
    P = case["num_pages"]
    move = np.random.default_rng(9).permutation(P)
    c2 = torch.zeros_like(cache_d)
    c2[torch.as_tensor(move, device=dev)] = cache_d
    case_m = dict(case)
    case_m["pt"] = np.where(case["pt"] >= 0, move[np.maximum(case["pt"], 0)], -1).astype(np.int32)
    o2, l2 = gpu_decode(case_m, c2, dev, smla)
    assert np.array_equal(o2, base_o) and np.array_equal(l2, base_l)
    # permute the lists
    case_p = dict(case)
    case_p["topk"] = case["topk"][:, np.random.default_rng(10).permutation(case["topk"].shape[1])]
    o3, l3 = gpu_decode(case_p, cache_d, dev, smla)
    # a different order regroups rows into tiles, which moves the running max
    # each weight is rounded to f16 against: each weight moves by <= 2^-11
    # relative, so out moves by <= ~2^-10 relative and lse by <= ~2^-11
    assert rel_l2(o3, base_o.astype(np.float64)) < 1e-3
    assert np.max(np.abs(l3 - base_l)) < 1e-3


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _ascending_lists(case, cache_o, qmul):
    """q times qmul, and every list reordered by ascending score (max over
    heads), so that later tiles keep passing the running max by a wide
    margin.  Returns the new case and the score of each list entry [B,H,K]
    in log2 units."""
    q = _bf16_to_f32(case["q"]) * np.float32(qmul)
    case = dict(case, q=wl.bf16_bits(torch.from_numpy(q).to(torch.bfloat16)))
    qf = _bf16_to_f32(case["q"]).astype(np.float64)
    rb = cache_o.shape[2]
    vals = (oracle.dequant_rows if rb == oracle.ROW_BYTES else oracle.dequant_rows_fp8)(
        cache_o.reshape(-1, rb))
    tk = case["topk"].copy()
    B, H, K = qf.shape[0], qf.shape[1], tk.shape[1]
    scores = np.full((B, H, K), -np.inf)
    for b in range(B):
        idx = tk[b][tk[b] >= 0].astype(np.int64)
        rows = case["pt"][b][idx // 64].astype(np.int64) * 64 + idx % 64
        sc = qf[b] @ vals[rows].T * case["scale"] / np.log(2.0)
        order = np.argsort(sc.max(axis=0), kind="stable")
        tk[b, :idx.size] = idx[order]
        tk[b, idx.size:] = -1
        scores[b, :, :idx.size] = sc[:, order]
    case["topk"] = tk
    return case, scores


def _max_moves(scores, splits, slack=8.0):
    """Tiles of 64 (per split of the list) whose maximum passes the maximum
    of the earlier tiles of the same split by more than the slack."""
    B, H, K = scores.shape
    per = -(-K // splits)
    moves = 0
    for b in range(B):
        for sp in range(splits):
            seg = scores[b, :, sp * per:(sp + 1) * per]
            run = None
            for t0 in range(0, seg.shape[1], 64):
                tm = seg[:, t0:t0 + 64].max(axis=1)
                if run is not None:
                    moves += int(np.any(tm > run + slack))
                    run = np.maximum(run, tm)
                else:
                    run = tm
    return moves


def _plan(batch, heads, topk, fp8=False, tokens=1):
    """(workgroups sharing a list, splits) of the library's plan."""
    return decode_plan(batch, heads, topk, fp8, tokens)[:2]


def _shared_pages_case(batch, heads, pages, topk, seed):
    """batch sequences whose page tables are permutations of the same
    `pages` physical pages (one shared context), each with its own query and
    its own top-k list: many sequences at the cost of quantising few rows."""
    rng = np.random.default_rng(seed)
    x = torch.randn((pages * 64, 576), generator=torch.Generator().manual_seed(seed))
    x[:, rng.choice(576, 8, replace=False)] *= 8
    bits = wl.bf16_bits(x.to(torch.bfloat16))
    pt = np.stack([rng.permutation(pages) for _ in range(batch)]).astype(np.int32)
    L = pages * 64
    tk = np.stack([rng.choice(L, topk, replace=False) for _ in range(batch)]).astype(np.int32)
    q = wl.bf16_bits(torch.randn((batch, heads, 576),
                                 generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16))
    return dict(q=q, rows=[bits], pt=pt, num_pages=pages, lens=np.full(batch, L, dtype=np.int64),
                topk=tk, scale=1.0 / np.sqrt(576.0))


@pytest.mark.parametrize("batch,heads", [(128, 16), (64, 64)])
def test_decode_running_max_moves(dev, smla, batch, heads):
    note("decode ascending lists B=%d H=%d" % (batch, heads))
    case = _shared_pages_case(batch, heads, 40, 2048, seed=40 + heads)
    cache_o = oracle_cache(case)
    case, scores = _ascending_lists(case, cache_o, 16.0)
    units, splits = _plan(batch, heads, 2048)
    # the re-weight path runs, on average, at least once per workgroup
    assert _max_moves(scores, splits) >= units * splits
    cache_d = gpu_cache(case, dev, smla)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)


def test_decode_64_heads_long_splits(dev, smla):
    """128 queries of 64 heads: 256 workgroups of one split of 2048 entries,
    32 tiles per workgroup, so the tile pipeline runs long and no merge
    follows; every query and head against the oracle."""
    note("decode B=128 H=64 K=2048 (long splits)")
    case = _shared_pages_case(128, 64, 40, 2048, seed=88)
    assert _plan(128, 64, 2048) == (256, 1)
    cache_d = gpu_cache(case, dev, smla)
    cache_o = oracle_cache(case)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)


def test_split_partials_f16_error_share(dev, smla):
    """A split stores its normalised partial in f16 (one rounding after the
    fp32 accumulation).
    The oracle decodes each split's slice of the list exactly; merging those
    exact partials reproduces the oracle's decode (which pins the split
    boundaries), and merging their f16 roundings gives the result an exact
    kernel with f16 partials would return.  Its distance from the exact
    decode is the partials' error, bounded per element by 2^-11 times the
    largest partial magnitude; its share of the GPU's error is reported.
    (8 queries of 64 heads take 16-head groups and 8 splits of 256.)"""
    B, H, K = 8, 64, 2048
    note("decode B=%d H=%d K=%d: f16 partials' error share" % (B, H, K))
    case = small_case(B, H, [4096] * B, K, seed=77)
    units, splits = _plan(B, H, K)
    assert (units, splits) == (32, 8)
    per = -(-K // splits)
    cache_o = oracle_cache(case)
    cache_d = gpu_cache(case, dev, smla)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    parts = []
    for sp in range(splits):
        cs = dict(case)
        cs["topk"] = np.ascontiguousarray(case["topk"][:, sp * per:(sp + 1) * per])
        parts.append(oracle_decode(cs, cache_o))
    po = np.stack([p[0] for p in parts])          # [S, B, H, 512] normalised partials
    pl = np.stack([p[1] for p in parts])          # [S, B, H] natural-log sums
    w = np.exp(pl - np.logaddexp.reduce(pl, axis=0))[..., None]   # split weights, sum 1
    exact = (w * po).sum(0)
    rounded = (w * po.astype(np.float16).astype(np.float64)).sum(0)
    assert rel_l2(exact, ref_o) < 1e-12
    # |f16(x) - x| <= 2^-11 |x| (2^-25 below f16's normal range); the weights
    # are a convex combination
    bound = 2.0 ** -11 * np.abs(po).max(0) + 2.0 ** -24
    assert (np.abs(rounded - exact) <= bound).all()
    e_part, e_gpu = rel_l2(rounded, ref_o), rel_l2(out, ref_o)
    note("  f16 partials rel_l2 %.3e, GPU rel_l2 %.3e: share %.2f" % (e_part, e_gpu, e_part / e_gpu))
    check_parity(out, ref_o, lse, ref_l)
    # the partials' rounding is one rounding among the path's f16 roundings
    # (operands, weights): it cannot exceed the bar by itself
    assert e_part <= OUT_TOL / 10


# --------------------------------------------------------------------------
# full-size workloads: all queries on the GPU, sampled sequences on the oracle
# --------------------------------------------------------------------------

def _full_workload_check(dev, smla, name, sample, seed=0, fmt="nvfp4"):
    w = wl.WORKLOADS[name]
    rb = oracle.ROW_BYTES if fmt == "nvfp4" else oracle.FP8_ROW_BYTES
    quant = oracle.quant_rows if fmt == "nvfp4" else oracle.quant_rows_fp8
    lens = wl.context_lengths(w, seed)
    pt, num_pages = wl.build_page_table(w, lens, seed)
    note("full %s %s: %d pages (%.2f GB)" % (name, fmt, num_pages, num_pages * 64 * rb / 1e9))
    cache = torch.zeros((num_pages, 64, rb), dtype=torch.uint8, device=dev)
    if fmt == "nvfp4":
        append = lambda rows, slots: smla.kv_quant_append(rows, slots, cache)
        decode = smla.sparse_mla_decode
    else:
        append = lambda rows, slots: smla.kv_quant_append_fp8(rows, slots, cache)
        decode = smla.sparse_mla_decode_fp8
    wl.fill_cache(w, seed, lens, pt, append, dev, tail=w.append_tail)
    if w.append_tail:
        rows, slots = wl.tail_rows(w, seed, lens, pt, dev, w.append_tail)
        note("  append %d tail rows" % rows.shape[0])
        append(rows, slots)
    tk = wl.topk_indices(w, lens, seed)
    q = wl.queries(w, seed, device=dev)
    note("  decode")
    out, lse = decode(q, cache, torch.as_tensor(pt, device=dev),
                      torch.as_tensor(lens.astype(np.int32), device=dev),
                      torch.as_tensor(tk, device=dev), w.softmax_scale)
    torch.cuda.synchronize(dev)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    qbits = wl.bf16_bits(q)
    flat = cache.view(-1, rb)
    worst = 0.0
    for b in sample:
        sel = tk[b][tk[b] >= 0].astype(np.int64)
        rows = wl.rows_at(w, seed, b, sel, device=dev)
        rbits = wl.bf16_bits(rows)
        mine = quant(rbits)
        slots = wl.slots_for(pt, b, 0, int(lens[b]))[sel].astype(np.int64)
        got_bytes = flat[torch.as_tensor(slots, device=dev)].cpu().numpy()
        assert np.array_equal(got_bytes, mine), "cache bytes differ for sequence %d" % b
        # the oracle on the selected rows alone, in list order
        n = sel.size
        mini = np.zeros(((n + 63) // 64, 64, rb), dtype=np.uint8)
        mini.reshape(-1, rb)[:n] = mine
        ro, rl = oracle.sparse_mla_decode(qbits[b:b + 1], mini,
                                          np.arange((n + 63) // 64, dtype=np.int32)[None],
                                          np.array([n]), np.arange(n, dtype=np.int32)[None],
                                          w.softmax_scale)
        e_out = check_parity(out[b:b + 1], ro, lse[b:b + 1], rl, "seq %d" % b)[0]
        worst = max(worst, e_out)
    del cache
    torch.cuda.empty_cache()
    return worst


def test_full_tp4(dev, smla):
    _full_workload_check(dev, smla, "tp4", sample=[0, 17, 31])


def test_full_allheads(dev, smla):
    _full_workload_check(dev, smla, "allheads", sample=[0, 40, 63])


def test_full_ragged(dev, smla):
    w = wl.WORKLOADS["ragged"]
    lens = wl.context_lengths(w, 0)
    short = [int(np.argmin(lens))]
    _full_workload_check(dev, smla, "ragged", sample=short + [0, 127])


def test_full_million(dev, smla):
    _full_workload_check(dev, smla, "million", sample=[0, 7])


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_decode_ignores_unselected_nan_row(dev, smla, fmt):
    """The last tile is padded with row 0 of page 0; when that row is not
    selected its bytes (here all 0xFF: NaN scales, NaN E4M3 values) must not
    reach the output."""
    note("decode with a NaN row 0 of page 0 (%s)" % fmt)
    case = small_case(3, 64, [700, 300, 150], 2048, seed=61)
    rb = 352 if fmt == "nvfp4" else 576
    for b in range(3):
        L = int(case["lens"][b])
        owner = [t for t in range(0, L, 64) if case["pt"][b][t // 64] == 0]
        for t in owner:                                     # token on page 0, row 0
            case["topk"][b][case["topk"][b] == t] = -1
    assert all((case["topk"][b] >= 0).sum() % 64 for b in range(3))     # ragged last tiles
    cache_o = oracle_cache(case, fmt)
    cache_o[0, 0, :] = 0xFF
    cache_d = gpu_cache(case, dev, smla, fmt)
    cache_d[0, 0, :] = 0xFF
    assert np.array_equal(cache_d.cpu().numpy(), cache_o)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    assert np.isfinite(ref_o).all()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    check_parity(out, ref_o, lse, ref_l)


def test_decode_max_batch(dev, smla):
    """The largest batch the ABI takes: 65,535 sequences of 64 heads, so that
    element offsets into q, out and lse pass 2^31; each sequence one page
    (of a global permutation) and a list of its 64 tokens with padding;
    sampled sequences against the oracle."""
    B, H, K, L = 65535, 64, 80, 64
    note("decode max batch B=%d H=%d" % (B, H))
    g = torch.Generator(device=dev)
    g.manual_seed(123)
    perm = torch.randperm(B + 3, generator=g, device=dev)[:B].to(torch.int32)
    pt = perm[:, None].contiguous()                                  # page of sequence b
    rows = torch.randn((B * L, 576), generator=g, device=dev).to(torch.bfloat16)
    slots = (pt.to(torch.int64) * 64 + torch.arange(64, device=dev)[None, :]).reshape(-1)
    cache = torch.zeros((B + 3, 64, 352), dtype=torch.uint8, device=dev)
    smla.kv_quant_append(rows, slots.to(torch.int32), cache)
    q = torch.randn((B, H, 576), generator=g, device=dev).to(torch.bfloat16)
    order = torch.argsort(torch.rand((B, L), generator=g, device=dev), dim=1).to(torch.int32)
    tk = torch.full((B, K), -1, dtype=torch.int32, device=dev)
    tk[:, 3:3 + L] = order
    sl = torch.full((B,), L, dtype=torch.int32, device=dev)
    out, lse = smla.sparse_mla_decode(q, cache, pt, sl, tk, 1.0 / np.sqrt(576.0))
    torch.cuda.synchronize(dev)
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    for b in (0, 1, 32767, B - 2, B - 1):
        rb = wl.bf16_bits(rows[b * L:(b + 1) * L])
        mini = oracle.quant_rows(rb).reshape(1, 64, 352)
        got_bytes = cache[int(pt[b, 0])].cpu().numpy()
        assert np.array_equal(got_bytes, mini[0]), "cache bytes differ for sequence %d" % b
        ro, rl = oracle.sparse_mla_decode(wl.bf16_bits(q[b:b + 1]), mini, np.zeros((1, 1), np.int32),
                                          np.array([L]), tk[b:b + 1].cpu().numpy(), 1.0 / np.sqrt(576.0))
        check_parity(out[b:b + 1].cpu().numpy(), ro, lse[b:b + 1].cpu().numpy(), rl, "seq %d" % b)
    del rows, q, out, lse, cache
    torch.cuda.empty_cache()


def test_decode_workspace_reuse_across_shapes(dev, smla):
    """One workspace serves calls of different shapes and both row formats
    in a row: each result equals the one a fresh workspace gives (bit for
    bit: the merge order is fixed)."""
    note("decode workspace reuse across shapes")
    from cases import gpu_cache, small_case
    shapes = [(2, 64, [5000, 1500], 2048), (1, 16, [4096], 256), (4, 16, [2500, 2500, 90, 700], 2048),
              (5, 64, [2100, 300, 64, 1, 4000], 2048), (1, 64, [70000], 2048), (3, 16, [3000, 777, 64], 512),
              (128, 16, [3000] * 128, 2048)]
    need = max(max(smla.decode_workspace_bytes(b, h, k), smla.decode_workspace_bytes_fp8(b, h, k))
               for b, h, _, k in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev)
    for trial, (batch, heads, lens, topk) in enumerate(shapes * 2):
        case = small_case(batch, heads, lens, topk, seed=300 + trial)
        fp8 = trial % 3 == 2
        cache_d = gpu_cache(case, dev, smla, fmt="fp8" if fp8 else "nvfp4")
        fn, wsb = ((smla.sparse_mla_decode_fp8, smla.decode_workspace_bytes_fp8) if fp8
                   else (smla.sparse_mla_decode, smla.decode_workspace_bytes))
        args = (to_dev_bf16(case["q"], dev), cache_d, torch.as_tensor(case["pt"], device=dev),
                torch.as_tensor(case["lens"].astype(np.int32), device=dev),
                torch.as_tensor(case["topk"], device=dev), case["scale"])
        o1, l1 = fn(*args, workspace=ws)
        fresh = torch.full((max(wsb(batch, heads, topk), 256),), 0x5A, dtype=torch.uint8, device=dev)
        o2, l2 = fn(*args, workspace=fresh)
        torch.cuda.synchronize(dev)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), trial


def test_binding_rejects_misshaped_outputs_and_foreign_workspace(dev, smla):
    """A caller-supplied out, lse or workspace that does not fit the call is
    refused with ValueError before anything is launched (the buffers keep
    their contents)."""
    note("binding checks of out, lse and workspace")
    case = small_case(2, 64, [3000, 1000], 512, seed=77)
    cache_d = gpu_cache(case, dev, smla)
    q = to_dev_bf16(case["q"], dev)
    pt = torch.as_tensor(case["pt"], device=dev)
    sl = torch.as_tensor(case["lens"].astype(np.int32), device=dev)
    tk = torch.as_tensor(case["topk"], device=dev)
    bad_out = torch.full((2, 16, 512), 7.0, device=dev)          # 16 heads for a 64-head q
    bad_lse = torch.full((2, 63), 7.0, device=dev)
    good_out = torch.full((2, 64, 512), 7.0, device=dev)
    good_lse = torch.full((2, 64), 7.0, device=dev)
    calls = [dict(out=bad_out), dict(lse=bad_lse), dict(out=good_out, lse=bad_lse),
             dict(workspace=torch.zeros(1 << 20, dtype=torch.uint8)),               # host memory
             dict(workspace=torch.zeros((1 << 20, 2), dtype=torch.uint8, device=dev)[:, 0])]
    for kw in calls:
        with pytest.raises(ValueError):
            smla.sparse_mla_decode(q, cache_d, pt, sl, tk, case["scale"], **kw)
    qm, tkm = q[:, None].contiguous(), tk[:, None].contiguous()
    for kw in (dict(out=good_out), dict(lse=good_lse),
               dict(workspace=torch.zeros(1 << 20, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            smla.sparse_mla_decode_mtp(qm, cache_d, pt, sl, tkm, case["scale"], **kw)
    torch.cuda.synchronize(dev)
    for t in (bad_out, bad_lse, good_out, good_lse):
        assert bool((t == 7.0).all())
    # the same buffers, shaped right, are accepted
    out, lse = smla.sparse_mla_decode(q, cache_d, pt, sl, tk, case["scale"], out=good_out,
                                      lse=good_lse)
    torch.cuda.synchronize(dev)
    ref_o, ref_l = oracle_decode(case, oracle_cache(case))
    check_parity(out.cpu().numpy(), ref_o, lse.cpu().numpy(), ref_l)
