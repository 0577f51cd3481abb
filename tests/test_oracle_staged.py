"""CPU pins of the oracle's staged path (the ablation of the fused kernel).

"Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", section
"A kernel that reads four bits directly" (the staged-vs-native figure and the
paragraph before it), and the launch post's account of its first
implementation: a gather kernel turns the selected NVFP4 rows into a
temporary 576-byte FP8 copy in HBM, and an FP8 attention kernel reads that
copy.  The copy is the lean FP8 row, each value the E4M3 value nearest the
decoded NVFP4 value.

Pinned against: the rows decoded by a library-based decoder (torch's E4M3
table and the e2m1 magnitudes) and re-encoded by torch's float8_e4m3fn cast;
the entry rules of the decode; and a closed form -- when every decoded value
is already an E4M3 value the copy is lossless, so the staged result equals
the fused one exactly.
"""
import math

import numpy as np
import torch

import oracle
import workloads as wl
from test_oracle_decode import make_case
from test_oracle_format import _independent_decode, torch_e4m3_encode

SCALE = 1.0 / math.sqrt(576)


def _library_stage(nvfp4_rows: np.ndarray) -> np.ndarray:
    vals = _independent_decode(nvfp4_rows)                  # exact values, fp64
    clipped = np.clip(vals, -448.0, 448.0)                  # saturation (torch gives NaN past 464)
    return torch_e4m3_encode(clipped.ravel()).reshape(vals.shape)


def test_staged_rows_match_library_reencode():
    case = make_case(B=2, H=2, lens=(300, 200), seed=21)
    rng = np.random.default_rng(22)
    K = 150
    topk = np.stack([rng.choice(300, K, replace=False),
                     np.concatenate([rng.choice(200, 100, replace=False), np.full(50, -1)])])
    topk = topk.astype(np.int32)
    staged, st = oracle.stage_rows_fp8(case["cache"], case["pt"], case["lens"], topk)
    kpad = 192
    assert staged.shape == (2 * kpad // 64, 64, 576)
    flat = staged.reshape(-1, 576)
    for b in range(2):
        for e in range(K):
            t = int(topk[b, e])
            if t < 0:
                assert st[b, e] == -1
                assert not flat[b * kpad + e].any()
                continue
            assert st[b, e] == e
            slot = int(case["pt"][b][t // 64]) * 64 + t % 64
            src = case["cache"].reshape(-1, 352)[slot][None]
            assert np.array_equal(flat[b * kpad + e], _library_stage(src)[0]), (b, e)


def test_staged_saturates_large_products():
    # scale 448 (code 0x7E) times e2m1 6 is 2688: the copy holds 448
    row = np.zeros((1, 64, 352), dtype=np.uint8)
    row[0, 0, :256] = 0x77                                  # every nibble +6
    row[0, 0, 256:288] = 0x7E
    row[0, 0, 0] = 0xF7                                     # element 1 is -6
    pt = np.zeros((1, 1), dtype=np.int32)
    staged, st = oracle.stage_rows_fp8(row, pt, np.array([64]), np.array([[0]], dtype=np.int32))
    r = staged.reshape(-1, 576)[0]
    assert st[0, 0] == 0
    assert r[0] == 0x7E and r[1] == 0xFE and (r[2:512] == 0x7E).all()
    assert (r[512:] == 0).all()


def test_staged_entry_rules_and_untouched_rows():
    case = make_case(B=2, H=2, lens=(130, 64), seed=23)
    pt = case["pt"].copy()
    pt[0, 1] = case["cache"].shape[0] + 9                   # tokens 64..127 on a bad page
    topk = np.array([[5, -1, 129, 130, 70, 10 ** 6, -7, 127],
                     [63, 64, 0, -1, 2, 2, 65, 1]], dtype=np.int32)
    init = np.full((2 * 64 // 64, 64, 576), 0x5A, dtype=np.uint8)
    staged, st = oracle.stage_rows_fp8(case["cache"], pt, case["lens"], topk, staged=init)
    want = np.array([[0, -1, 2, -1, -1, -1, -1, -1],
                     [0, -1, 2, -1, 4, 5, -1, 7]], dtype=np.int32)
    assert np.array_equal(st, want)
    flat = staged.reshape(-1, 576)
    for b in range(2):
        for e in range(8):
            if want[b, e] < 0:
                assert (flat[b * 64 + e] == 0x5A).all()
            else:
                assert not (flat[b * 64 + e] == 0x5A).all()
    assert (flat[8:64] == 0x5A).all() and (flat[72:] == 0x5A).all()


def test_lossless_copy_gives_the_fused_result():
    """Rows whose scales are powers of two in [2^-6, 2^6] decode to values
    e2m1 x 2^j, all of them E4M3 values: the staged attention then equals the
    fused attention bit for bit."""
    rng = np.random.default_rng(24)
    B, H, L = 2, 3, 256
    pages = L // 64
    cache = np.zeros((B * pages, 64, 352), dtype=np.uint8)
    flat = cache.reshape(-1, 352)
    flat[:, :256] = rng.integers(0, 256, size=(B * L, 256))
    pow2_codes = np.array([(e + 7) << 3 for e in range(-6, 7)], dtype=np.uint8)
    flat[:, 256:288] = rng.choice(pow2_codes, size=(B * L, 32))
    rope = rng.integers(0, 256, size=(B * L, 64)).astype(np.uint8)
    rope[(rope & 0x7F) == 0x7F] = 0x7E
    flat[:, 288:] = rope
    pt = np.arange(B * pages, dtype=np.int32).reshape(B, pages)
    lens = np.full(B, L, dtype=np.int64)
    topk = np.stack([rng.choice(L, 100, replace=False) for _ in range(B)]).astype(np.int32)
    q = wl.bf16_bits(torch.randn((B, H, 576), generator=torch.Generator().manual_seed(25))
                     .to(torch.bfloat16))
    o1, l1 = oracle.sparse_mla_decode(q, cache, pt, lens, topk, SCALE)
    staged, st = oracle.stage_rows_fp8(cache, pt, lens, topk)
    spt, slen = oracle.staged_tables(B, topk.shape[1])
    o2, l2 = oracle.sparse_mla_decode(q, staged, spt, slen, st, SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lossy_copy_stays_close_to_the_fused_result():
    case = make_case(B=2, H=4, lens=(400, 333), seed=26)
    rng = np.random.default_rng(27)
    topk = np.stack([rng.choice(400, 256, replace=False),
                     rng.choice(333, 256, replace=False)]).astype(np.int32)
    o1, l1 = oracle.sparse_mla_decode(case["q"], case["cache"], case["pt"], case["lens"], topk,
                                      SCALE)
    staged, st = oracle.stage_rows_fp8(case["cache"], case["pt"], case["lens"], topk)
    spt, slen = oracle.staged_tables(2, 256)
    o2, l2 = oracle.sparse_mla_decode(case["q"], staged, spt, slen, st, SCALE)
    # E4M3 keeps 3 mantissa bits: each value moves by at most 2^-4 relative
    rel = np.linalg.norm(o2 - o1) / np.linalg.norm(o1)
    assert 0 < rel < 2 ** -4
    assert np.max(np.abs(l2 - l1)) < 0.5


def test_staged_skips_entries_past_the_page_table():
    """seq_lens past max_pages * 64: an entry whose page-table column does not
    exist is unusable (staged_topk -1, its staged row untouched), like -1."""
    case = make_case(B=2, H=2, lens=(250, 200), seed=25)
    max_pages = 2                                        # tokens 0..127 have a page
    narrow = np.ascontiguousarray(case["pt"][:, :max_pages])
    topk = np.array([[5, 130, 127, 200, 249, 64],
                     [128, 0, 199, 63, 150, 100]], dtype=np.int32)
    init = np.full((2, 64, 576), 0x5A, dtype=np.uint8)
    staged, st = oracle.stage_rows_fp8(case["cache"], narrow, case["lens"], topk, staged=init)
    want = np.where(topk < 64 * max_pages, np.arange(6)[None, :], -1)
    assert np.array_equal(st, want)
    flat = staged.reshape(-1, 576)
    for b in range(2):
        for e in range(6):
            t = int(topk[b, e])
            if want[b, e] < 0:
                assert (flat[b * 64 + e] == 0x5A).all()
            else:
                slot = int(narrow[b][t // 64]) * 64 + t % 64
                src = case["cache"].reshape(-1, 352)[slot][None]
                assert np.array_equal(flat[b * 64 + e], _library_stage(src)[0]), (b, e)
