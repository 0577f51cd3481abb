"""GPU parity of the lean FP8 row variant against the CPU oracle (through the C ABI).

Same bars as the NVFP4 path: cache bytes bit-exact; decode out within 2e-2
relative L2 over the whole [B,H,512] tensor and lse within 1e-3 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from cases import (check_parity, gpu_cache, gpu_decode, note, oracle_cache, oracle_decode,
                   small_case, to_dev_bf16)
from test_gpu_parity import (DECODE_CASES, _ascending_lists, _plan,
                             _full_workload_check, _max_moves, _shared_pages_case)

pytestmark = pytest.mark.gpu

RB = oracle.FP8_ROW_BYTES


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
    cache = torch.zeros((pages, 64, RB), dtype=torch.uint8, device=dev)
    slots = torch.arange(n, dtype=torch.int32, device=dev)
    smla.kv_quant_append_fp8(to_dev_bf16(bits, dev), slots, cache)
    torch.cuda.synchronize(dev)
    return cache.view(-1, RB)[:n].cpu().numpy()


def test_fp8_quant_every_bf16_in_every_position(dev, smla):
    """Every finite BF16 value reaches every one of the 576 positions: covers
    rounding ties, subnormal codes and saturation."""
    note("fp8 quant every finite bf16 value")
    b = np.arange(65536, dtype=np.uint32)
    finite = b[((b >> 7) & 0xFF) != 0xFF]
    n = finite.size
    r = np.arange(n, dtype=np.int64)[:, None]
    p = np.arange(576, dtype=np.int64)[None, :]
    bits = finite[(r + 97 * p) % n].astype(np.uint16)        # row r, position p
    assert all(np.unique(bits[:, j]).size == n for j in (0, 300, 511, 512, 575))
    got = _append_and_read(smla, dev, bits)
    want = oracle.quant_rows_fp8(bits)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


def test_fp8_quant_random_rows_bit_exact(dev, smla):
    note("fp8 quant random rows n=5000")
    g = torch.Generator().manual_seed(11)
    x = torch.randn((5000, 576), generator=g)
    x[:1000] *= 200.0
    x[1000:2000] *= 1e-3
    x[2000:2100] *= 1e4
    bits = wl.bf16_bits(x.to(torch.bfloat16))
    got = _append_and_read(smla, dev, bits)
    want = oracle.quant_rows_fp8(bits)
    assert np.array_equal(got, want), np.argwhere(got != want)[:10]


def test_fp8_quant_slot_mapping_skips_and_leaves_others(dev, smla):
    note("fp8 quant slot mapping")
    n = 300
    bits = wl.bf16_bits(torch.randn((n, 576), generator=torch.Generator().manual_seed(13))
                        .to(torch.bfloat16))
    pages = 6
    slots = np.random.default_rng(14).permutation(pages * 64)[:n].astype(np.int32)
    slots[::7] = -1
    slots[5] = pages * 64
    slots[6] = 2 ** 31 - 1
    cache = torch.full((pages, 64, RB), 0xAB, dtype=torch.uint8, device=dev)
    smla.kv_quant_append_fp8(to_dev_bf16(bits, dev), torch.as_tensor(slots, device=dev), cache)
    torch.cuda.synchronize(dev)
    want = np.full((pages, 64, RB), 0xAB, dtype=np.uint8)
    oracle.kv_quant_append_fp8(bits, slots, want)
    assert np.array_equal(cache.cpu().numpy(), want)


@pytest.mark.parametrize("batch,heads,lens,topk,kw", DECODE_CASES,
                         ids=["B%d_H%d_K%d_%d" % (c[0], c[1], c[3], i)
                              for i, c in enumerate(DECODE_CASES)])
def test_fp8_decode_matches_oracle(dev, smla, batch, heads, lens, topk, kw):
    case = small_case(batch, heads, lens, topk, seed=batch * 100 + topk + 1, **kw)
    note("fp8 decode B=%d H=%d lens=%s K=%d %s" % (batch, heads, lens, topk, kw))
    cache_d = gpu_cache(case, dev, smla, "fp8")
    cache_o = oracle_cache(case, "fp8")
    assert np.array_equal(cache_d.cpu().numpy(), cache_o)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)


def test_fp8_decode_empty_selections(dev, smla):
    note("fp8 decode empty selections")
    case = small_case(3, 64, [100, 50, 10], 64, seed=15)
    case["topk"][:] = -1
    case["topk"][1, :5] = [50, 51, 99, -3, 10 ** 6]
    out, lse = gpu_decode(case, gpu_cache(case, dev, smla, "fp8"), dev, smla)
    assert not out.any()
    assert np.isneginf(lse).all()


def test_fp8_decode_invariances(dev, smla):
    """Page relocation is bit-identical, and so is a second call."""
    note("fp8 decode invariances")
    case = small_case(2, 64, [2000, 900], 1024, seed=18, pad=200)
    cache_d = gpu_cache(case, dev, smla, "fp8")
    base_o, base_l = gpu_decode(case, cache_d, dev, smla)
    again_o, again_l = gpu_decode(case, cache_d, dev, smla)
    assert np.array_equal(again_o, base_o) and np.array_equal(again_l, base_l)
    P = case["num_pages"]
    move = np.random.default_rng(19).permutation(P)
    c2 = torch.zeros_like(cache_d)
    c2[torch.as_tensor(move, device=dev)] = cache_d
    case_m = dict(case)
    case_m["pt"] = np.where(case["pt"] >= 0, move[np.maximum(case["pt"], 0)], -1).astype(np.int32)
    o2, l2 = gpu_decode(case_m, c2, dev, smla)
    assert np.array_equal(o2, base_o) and np.array_equal(l2, base_l)


@pytest.mark.parametrize("batch,heads", [(128, 16), (64, 64)])
def test_fp8_decode_running_max_moves(dev, smla, batch, heads):
    note("fp8 decode ascending lists B=%d H=%d" % (batch, heads))
    case = _shared_pages_case(batch, heads, 40, 2048, seed=50 + heads)
    cache_o = oracle_cache(case, "fp8")
    case, scores = _ascending_lists(case, cache_o, 16.0)
    # an FP8 workgroup covers at most 1024 list entries, so the list is cut
    # into at least two splits
    units, splits = _plan(batch, heads, 2048, fp8=True)
    assert _max_moves(scores, splits) >= units * splits
    cache_d = gpu_cache(case, dev, smla, "fp8")
    assert np.array_equal(cache_d.cpu().numpy(), cache_o)
    out, lse = gpu_decode(case, cache_d, dev, smla)
    ref_o, ref_l = oracle_decode(case, cache_o)
    check_parity(out, ref_o, lse, ref_l)


def test_fp8_full_tp4(dev, smla):
    _full_workload_check(dev, smla, "tp4", sample=[0, 31], fmt="fp8")


def test_fp8_full_allheads(dev, smla):
    _full_workload_check(dev, smla, "allheads", sample=[0, 63], fmt="fp8")
