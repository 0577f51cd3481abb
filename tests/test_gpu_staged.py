"""GPU parity of the staged path (gather-unpack to an FP8 copy, then FP8
decode) against the CPU oracle, through the C ABI.

Bars: the copy and its list bit-exact; out within 2e-2 relative L2 and lse
within 1e-3 absolute of the oracle's attention over its own copy.
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


def _dev_tables(case, dev):
    pt = torch.as_tensor(np.ascontiguousarray(case["pt"]), device=dev)
    sl = torch.as_tensor(np.ascontiguousarray(case["lens"].astype(np.int32)), device=dev)
    tk = torch.as_tensor(np.ascontiguousarray(case["topk"]), device=dev)
    return pt, sl, tk


def test_staged_every_nibble_scale_product(dev, smla):
    """Every e2m1 code times every finite E4M3 scale code (both signs), as
    cache bytes written directly: covers the re-encode's rounding, ties,
    subnormals, signed zeros and saturation (6 x 448 -> 448)."""
    note("staged: every nibble x scale product")
    scales = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    nrows = -(-scales.size // 32) + 2
    rng = np.random.default_rng(71)
    rows = np.zeros((64, 352), dtype=np.uint8)
    nib = np.tile(np.arange(16, dtype=np.uint8), 32)               # every code in every block
    for r in range(nrows):
        perm = np.concatenate([rng.permutation(16) for _ in range(32)]).astype(np.uint8)
        nn = nib[perm + np.repeat(np.arange(32) * 16, 16)] if r % 2 else nib
        rows[r, :256] = nn[0::2] | (nn[1::2] << 4)
        rows[r, 256:288] = np.resize(np.roll(scales, -32 * r), 32)
        rope = rng.integers(0, 256, size=64).astype(np.uint8)
        rope[(rope & 0x7F) == 0x7F] = 0x7E
        rows[r, 288:] = rope
    cache_np = rows[None].copy()
    pt_np = np.zeros((1, 1), dtype=np.int32)
    lens = np.array([64], dtype=np.int32)
    tk_np = np.arange(nrows, dtype=np.int32)[None]
    want, want_st = oracle.stage_rows_fp8(cache_np, pt_np, lens, tk_np)
    cache = torch.as_tensor(cache_np, device=dev)
    staged, st = smla.stage_rows_fp8(cache, torch.as_tensor(pt_np, device=dev),
                                     torch.as_tensor(lens, device=dev),
                                     torch.as_tensor(tk_np, device=dev))
    torch.cuda.synchronize(dev)
    assert np.array_equal(st.cpu().numpy(), want_st)
    got = staged.cpu().numpy().reshape(-1, 576)[:nrows]
    ref = want.reshape(-1, 576)[:nrows]
    bad = np.argwhere(got != ref)
    assert bad.size == 0, [(int(r), int(c), int(got[r, c]), int(ref[r, c])) for r, c in bad[:8]]


STAGE_CASES = [
    (1, 16, [4096], 256, {}),
    (3, 16, [3000, 777, 64], 512, dict(pad=100)),
    (2, 64, [5000, 1500], 2048, {}),
    (2, 16, [1000, 1000], 100, dict(dup=10, junk=5)),
    (2, 64, [333, 129], 17, dict(junk=3)),
    (6, 16, [64, 65, 127, 128, 129, 1], 64, {}),
]


@pytest.mark.parametrize("batch,heads,lens,topk,kw", STAGE_CASES,
                         ids=["B%d_H%d_K%d_%d" % (c[0], c[1], c[3], i)
                              for i, c in enumerate(STAGE_CASES)])
def test_staged_copy_and_decode_match_oracle(dev, smla, batch, heads, lens, topk, kw):
    case = small_case(batch, heads, lens, topk, seed=batch * 31 + topk, **kw)
    note("staged B=%d H=%d lens=%s K=%d %s" % (batch, heads, lens, topk, kw))
    cache_d = gpu_cache(case, dev, smla)
    cache_o = oracle_cache(case)
    pt, sl, tk = _dev_tables(case, dev)
    pp = -(-topk // 64)
    staged = torch.full((batch * pp, 64, 576), 0x5A, dtype=torch.uint8, device=dev)
    staged, st = smla.stage_rows_fp8(cache_d, pt, sl, tk, staged=staged)
    torch.cuda.synchronize(dev)
    init = np.full((batch * pp, 64, 576), 0x5A, dtype=np.uint8)
    want, want_st = oracle.stage_rows_fp8(cache_o, case["pt"], case["lens"], case["topk"],
                                          staged=init)
    assert np.array_equal(st.cpu().numpy(), want_st)
    got = staged.cpu().numpy()
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]
    # attention over the copy, as the staged path runs it
    q = to_dev_bf16(case["q"], dev)
    out, lse = smla.sparse_mla_decode_staged(q, cache_d, pt, sl, tk, case["scale"])
    torch.cuda.synchronize(dev)
    spt, ssl = oracle.staged_tables(batch, topk)
    ref_o, ref_l = oracle.sparse_mla_decode(case["q"], want, spt, ssl, want_st, case["scale"])
    check_parity(out.cpu().numpy(), ref_o, lse.cpu().numpy(), ref_l)


def test_staged_full_allheads_sampled(dev, smla):
    w = wl.WORKLOADS["allheads"]
    lens = wl.context_lengths(w, 0)
    pt_np, num_pages = wl.build_page_table(w, lens, 0)
    note("staged full allheads: %d pages" % num_pages)
    cache = torch.zeros((num_pages, 64, 352), dtype=torch.uint8, device=dev)
    wl.fill_cache(w, 0, lens, pt_np, lambda r, s: smla.kv_quant_append(r, s, cache), dev)
    tk_np = wl.topk_indices(w, lens, 0)
    q = wl.queries(w, 0, device=dev)
    pt = torch.as_tensor(pt_np, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    tk = torch.as_tensor(tk_np, device=dev)
    staged, st = smla.stage_rows_fp8(cache, pt, sl, tk)
    out, lse = smla.sparse_mla_decode_staged(q, cache, pt, sl, tk, w.softmax_scale)
    torch.cuda.synchronize(dev)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    qbits = wl.bf16_bits(q)
    K = w.topk
    for b in (0, 63):
        sel = tk_np[b][tk_np[b] >= 0].astype(np.int64)
        rows = oracle.quant_rows(wl.bf16_bits(wl.rows_at(w, 0, b, sel, device=dev)))
        n = sel.size
        mini = np.zeros(((n + 63) // 64, 64, 352), dtype=np.uint8)
        mini.reshape(-1, 352)[:n] = rows
        mpt = np.arange(mini.shape[0], dtype=np.int32)[None]
        mtk = np.full((1, K), -1, dtype=np.int32)
        mtk[0, :n] = np.arange(n)
        want, want_st = oracle.stage_rows_fp8(mini, mpt, np.array([n]), mtk)
        got = staged[b * K // 64:(b + 1) * K // 64].cpu().numpy().reshape(-1, 576)
        assert np.array_equal(got[:n], want.reshape(-1, 576)[:n]), "staged rows differ, seq %d" % b
        spt, ssl = oracle.staged_tables(1, K)
        ro, rl = oracle.sparse_mla_decode(qbits[b:b + 1], want, spt, ssl, want_st, w.softmax_scale)
        check_parity(out[b:b + 1], ro, lse[b:b + 1], rl, "seq %d" % b)
    del cache, staged
    torch.cuda.empty_cache()
