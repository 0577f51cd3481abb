"""CPU pins of the oracle's multi-token decode (MTP verification: the
accepted token and its drafts, "GLM-5.3 PCP/DCP long-context on H200",
section 4, MTP speculative decoding with three draft tokens).

Pinned against: dense causal attention by torch's SDPA (fp64) with an
explicit mask, over rows decoded without the oracle; T = 1 reducing to the
plain decode; and the causal rule (entries a token may not see change
nothing).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads as wl
from test_oracle_decode import decoded_logical, make_case
from test_oracle_format import bf16_bits_to_f64

SCALE = 1.0 / math.sqrt(576)


def test_full_lists_reduce_to_causal_dense_attention():
    T, H = 4, 3
    case = make_case(B=2, H=H, lens=(300, 150), seed=41)
    q = wl.bf16_bits(torch.randn((2, T, H, 576), generator=torch.Generator().manual_seed(42))
                     .to(torch.bfloat16))
    K = 300
    topk = np.full((2, T, K), -1, dtype=np.int32)
    topk[0, :, :300] = np.arange(300)
    topk[1, :, :150] = np.arange(150)
    out, lse = oracle.sparse_mla_decode_mtp(q, case["cache"], case["pt"], case["lens"], topk, SCALE)
    for b in range(2):
        L = int(case["lens"][b])
        Kd = torch.from_numpy(decoded_logical(case, b))                     # [L, 576]
        qq = torch.from_numpy(bf16_bits_to_f64(q[b]))                        # [T, H, 576]
        pos = torch.arange(L)[None, :]
        allowed = pos < (L - (T - 1 - torch.arange(T)))[:, None]             # [T, L]
        for h in range(H):
            o = F.scaled_dot_product_attention(qq[None, None, :, h, :], Kd[None, None],
                                               Kd[None, None, :, :512], attn_mask=allowed[None, None],
                                               scale=SCALE)[0, 0]
            s = SCALE * (qq[:, h, :] @ Kd.T)
            l = torch.logsumexp(s.masked_fill(~allowed, -math.inf), dim=-1)
            np.testing.assert_allclose(out[b, :, h], o.numpy(), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b, :, h], l.numpy(), rtol=1e-13, atol=1e-13)


def test_one_token_is_the_plain_decode():
    case = make_case(B=2, H=4, lens=(260, 200), seed=43)
    rng = np.random.default_rng(44)
    topk = np.stack([rng.choice(260, 128, replace=False),
                     rng.choice(200, 128, replace=False)]).astype(np.int32)
    o1, l1 = oracle.sparse_mla_decode(case["q"], case["cache"], case["pt"], case["lens"], topk, SCALE)
    o2, l2 = oracle.sparse_mla_decode_mtp(case["q"][:, None], case["cache"], case["pt"],
                                          case["lens"], topk[:, None], SCALE)
    assert np.array_equal(o1, o2[:, 0]) and np.array_equal(l1, l2[:, 0])


def test_entries_a_token_cannot_see_change_nothing():
    T = 3
    case = make_case(B=1, H=2, lens=(200,), seed=45)
    q = wl.bf16_bits(torch.randn((1, T, 2, 576), generator=torch.Generator().manual_seed(46))
                     .to(torch.bfloat16))
    rng = np.random.default_rng(47)
    base = rng.choice(197, 60, replace=False)
    topk = np.full((1, T, 64), -1, dtype=np.int32)
    for j in range(T):
        topk[0, j, :60] = base
        topk[0, j, 60:64] = [197, 198, 199, 196]          # the newest positions
    o1, l1 = oracle.sparse_mla_decode_mtp(q, case["cache"], case["pt"], case["lens"], topk, SCALE)
    # token j sees [0, 198 + j): drop what it cannot see
    vis = topk.copy()
    for j in range(T):
        row = vis[0, j]
        row[row >= 198 + j] = -1
    o2, l2 = oracle.sparse_mla_decode_mtp(q, case["cache"], case["pt"], case["lens"], vis, SCALE)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # and the last token, which sees everything, differs from the first
    assert not np.array_equal(o1[0, 0], o1[0, T - 1])
