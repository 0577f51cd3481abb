"""CPU pins of the oracle's lean FP8 row (576 E4M3 bytes per token, no scale).

The row is the FP8 row of the byte table in "Prime Inference: serving GLM-5.3
to agents is a KV-cache problem", section "Four bits per latent value: where
352 comes from" (576 B per row, kept in tests/golden/page_figures.json).  The
oracle is fixed against: that byte count, PyTorch's float8_e4m3fn (a library
routine) for every finite BF16 value, exact round trips of every E4M3 code,
and dense attention by torch's SDPA over rows decoded by the library.
"""
import json
import math
import os

import numpy as np
import torch

import oracle
import workloads as wl
from test_oracle_decode import library_attention
from test_oracle_format import (_f64_to_bf16_exact, all_finite_bf16, bf16_bits_to_f64,
                                torch_e4m3_encode, torch_e4m3_value)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
SCALE = 1.0 / math.sqrt(576)


def test_fp8_row_bytes_match_pages():
    rb = json.load(open(GOLDEN))["row_bytes"]
    total = rb["fp8_row"]["total"]
    assert total == rb["latent_values"] + rb["rope_values"] == 576
    assert oracle._load().oracle_fp8_row_bytes() == total
    assert oracle.quant_rows_fp8(np.zeros((1, 576), np.uint16)).shape == (1, total)


def test_fp8_row_encode_every_bf16_against_library():
    bits = all_finite_bf16()
    n = -(-bits.size // 576) * 576
    rows = np.concatenate([bits, bits[: n - bits.size]]).reshape(-1, 576)
    got = oracle.quant_rows_fp8(rows).ravel()
    x = bf16_bits_to_f64(rows.ravel())
    inside = np.abs(x) <= 464.0                 # torch gives NaN past the last midpoint
    assert np.array_equal(got[inside], torch_e4m3_encode(x[inside]))
    sat = np.where(np.signbit(x[~inside]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(got[~inside], sat)


def test_fp8_row_round_trip_every_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    rng = np.random.default_rng(5)
    rows = rng.choice(codes, size=(40, 576)).astype(np.uint8)
    rows[0, :codes.size] = codes                              # every finite code appears
    vals = oracle.dequant_rows_fp8(rows)
    assert np.array_equal(vals, torch_e4m3_value(rows))
    assert np.array_equal(oracle.quant_rows_fp8(_f64_to_bf16_exact(vals)), rows)


def test_fp8_row_layout_single_nonzero():
    for d in (0, 1, 255, 256, 511, 512, 575):
        x = np.zeros((1, 576), dtype=np.uint16)
        x[0, d] = 0x3F80                                      # bf16 1.0 -> E4M3 0x38
        want = np.zeros(576, dtype=np.uint8)
        want[d] = 0x38
        assert np.array_equal(oracle.quant_rows_fp8(x)[0], want), d


def test_fp8_append_slot_rules():
    cache = np.full((2, 64, 576), 0xAB, dtype=np.uint8)
    x = wl.bf16_bits(torch.randn((4, 576), generator=torch.Generator().manual_seed(3))
                     .to(torch.bfloat16))
    slots = np.array([5, -1, 128, 127], dtype=np.int32)      # 128 is one past the end
    assert oracle.kv_quant_append_fp8(x, slots, cache) == 2
    flat = cache.reshape(-1, 576)
    rows = oracle.quant_rows_fp8(x)
    assert np.array_equal(flat[5], rows[0]) and np.array_equal(flat[127], rows[3])
    others = np.ones(128, dtype=bool)
    others[[5, 127]] = False
    assert (flat[others] == 0xAB).all()


def test_fp8_decode_is_attention_over_library_decoded_rows():
    rng = np.random.default_rng(8)
    B, H, L, K = 2, 5, 300, 96
    pages = (L + 63) // 64
    pt = np.stack([rng.permutation(2 * pages)[:pages] for _ in range(B)]).astype(np.int32)
    cache = np.zeros((2 * pages, 64, 576), dtype=np.uint8)
    for b in range(B):
        x = torch.randn((L, 576), generator=torch.Generator().manual_seed(20 + b))
        x[:, :8] *= 8
        oracle.kv_quant_append_fp8(wl.bf16_bits(x.to(torch.bfloat16)),
                                   wl.slots_for(pt, b, 0, L), cache)
    q = wl.bf16_bits(torch.randn((B, H, 576), generator=torch.Generator().manual_seed(9))
                     .to(torch.bfloat16))
    topk = np.full((B, K), -1, dtype=np.int32)
    topk[0] = rng.choice(L, K, replace=False)
    topk[1, :50] = rng.choice(L, 50, replace=False)
    lens = np.full(B, L, dtype=np.int64)
    out, lse = oracle.sparse_mla_decode(q, cache, pt, lens, topk, SCALE)
    for b in range(B):
        sel = topk[b][topk[b] >= 0].astype(np.int64)
        slots = pt[b][sel // 64].astype(np.int64) * 64 + sel % 64
        kmat = torch_e4m3_value(cache.reshape(-1, 576)[slots])
        ref_o, ref_l = library_attention(q[b], kmat, SCALE)
        np.testing.assert_allclose(out[b], ref_o, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[b], ref_l, rtol=1e-13, atol=1e-13)
