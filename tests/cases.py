"""Helpers that build the same seeded inputs for the HIP path and the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as wl


def note(msg: str):
    """Name the case on stdout before a GPU step (survives a crash of the step)."""
    sys.stdout.write("[case] %s\n" % msg)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got.astype(np.float64) - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def worst_head_rel(got: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(got.astype(np.float64) - ref, axis=-1)
    r = np.linalg.norm(ref, axis=-1)
    return float(np.max(np.where(r > 0, d / np.maximum(r, 1e-300), d)))


# The parity bars.  OUT_TOL and LSE_TOL are the stated ones: relative L2 of
# out over the whole tensor, absolute error of lse.  HEAD_TOL is the same
# relative L2 per (query, head) row of out, set from the arithmetic: the
# GPU path's only rounding beyond fp32 summation order is the f16 softmax
# weight (and the f16 split partial), 2^-11 relative each, so a head's error
# stays near 1e-3 at worst; 5e-3 leaves headroom while a systematic error in
# one head group, split or token (a dropped tile, a wrong scale) still fails.
OUT_TOL = 2e-2
LSE_TOL = 1e-3
HEAD_TOL = 5e-3


def check_parity(got_o, ref_o, got_l, ref_l, what: str = ""):
    """Assert the three bars; returns (rel_l2, worst_head_rel, lse_err)."""
    e_out, e_worst, e_lse = rel_l2(got_o, ref_o), worst_head_rel(got_o, ref_o), lse_err(got_l, ref_l)
    note("  %s rel_l2 %.3e worst-head %.3e lse %.3e" % (what, e_out, e_worst, e_lse))
    assert np.isfinite(np.asarray(got_o)).all(), what
    assert e_out <= OUT_TOL, (what, e_out)
    assert e_worst <= HEAD_TOL, (what, e_worst)
    assert e_lse <= LSE_TOL, (what, e_lse)
    return e_out, e_worst, e_lse


def lse_err(got: np.ndarray, ref: np.ndarray) -> float:
    g = got.astype(np.float64)
    both_inf = np.isneginf(g) & np.isneginf(ref)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), "-inf pattern differs"
    d = np.where(both_inf, 0.0, np.abs(np.where(both_inf, 0, g) - np.where(both_inf, 0, ref)))
    return float(d.max()) if d.size else 0.0


def small_case(batch, heads, lens, topk, seed=0, pages="global", pad=None, dup=0,
               junk=0, outliers=True, extra_pages=2):
    """A small decode problem with every token row materialised.

    pad:  number of -1 entries to scatter into each list (after the valid ones)
    dup:  number of repeated valid indices per list
    junk: number of out-of-range entries (t >= L, t < -1) per list
    Returns a dict of numpy arrays (BF16 as uint16 bits)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    npg = [(int(L) + 63) // 64 for L in lens]
    num_pages = int(sum(npg)) + extra_pages
    perm = rng.permutation(num_pages) if pages == "global" else np.arange(num_pages)
    pt = np.full((batch, max(max(npg), 1)), -1, dtype=np.int32)
    off = 0
    for b in range(batch):
        pt[b, :npg[b]] = perm[off:off + npg[b]]
        off += npg[b]
    rows = []
    ch = rng.choice(576, 8, replace=False)
    for b in range(batch):
        x = torch.randn((int(lens[b]), 576), generator=torch.Generator().manual_seed(seed * 1000 + b))
        if outliers:
            x[:, ch] *= 8
        rows.append(wl.bf16_bits(x.to(torch.bfloat16)))
    q = wl.bf16_bits(torch.randn((batch, heads, 576),
                                 generator=torch.Generator().manual_seed(seed * 1000 + 999))
                     .to(torch.bfloat16))
    tk = np.full((batch, topk), -1, dtype=np.int32)
    for b in range(batch):
        L = int(lens[b])
        n = min(topk - (pad or 0) - dup - junk, L) if L > 0 else 0
        n = max(n, 0)
        sel = list(rng.choice(L, n, replace=False)) if n else []
        if dup and sel:
            sel += list(rng.choice(sel, dup))
        sel += [int(v) for v in rng.choice([L, L + 7, 10 ** 7, -2, -(2 ** 31)], junk)]
        sel = np.array(sel, dtype=np.int64)
        sel = sel[rng.permutation(sel.size)]
        slots = np.sort(rng.choice(topk, sel.size, replace=False))
        tk[b, slots] = sel.astype(np.int32)
    return dict(q=q, rows=rows, pt=pt, num_pages=num_pages, lens=lens, topk=tk,
                scale=1.0 / np.sqrt(576.0))


ROW_BYTES = {"nvfp4": oracle.ROW_BYTES, "fp8": oracle.FP8_ROW_BYTES}


def oracle_cache(case, fmt: str = "nvfp4") -> np.ndarray:
    """The case's rows appended by the oracle into a cache of the given row format."""
    cache = np.zeros((case["num_pages"], 64, ROW_BYTES[fmt]), dtype=np.uint8)
    append = oracle.kv_quant_append if fmt == "nvfp4" else oracle.kv_quant_append_fp8
    for b, bits in enumerate(case["rows"]):
        if bits.shape[0]:
            append(bits, wl.slots_for(case["pt"], b, 0, bits.shape[0]), cache)
    return cache


def gpu_cache(case, dev, smla, fmt: str = "nvfp4") -> torch.Tensor:
    """The case's rows appended by the library into a device cache."""
    cache = torch.zeros((case["num_pages"], 64, ROW_BYTES[fmt]), dtype=torch.uint8, device=dev)
    append = smla.kv_quant_append if fmt == "nvfp4" else smla.kv_quant_append_fp8
    for b, bits in enumerate(case["rows"]):
        if bits.shape[0]:
            slots = torch.as_tensor(wl.slots_for(case["pt"], b, 0, bits.shape[0]), device=dev)
            append(to_dev_bf16(bits, dev), slots, cache)
    return cache


def gpu_decode(case, cache_dev, dev, smla):
    """Decode through the library; the cache's row size picks the entry point."""
    q = to_dev_bf16(case["q"], dev)
    pt = torch.as_tensor(np.ascontiguousarray(case["pt"]), device=dev)
    sl = torch.as_tensor(np.ascontiguousarray(case["lens"].astype(np.int32)), device=dev)
    tk = torch.as_tensor(np.ascontiguousarray(case["topk"]), device=dev)
    fn = smla.sparse_mla_decode if cache_dev.shape[2] == oracle.ROW_BYTES \
        else smla.sparse_mla_decode_fp8
    out, lse = fn(q, cache_dev, pt, sl, tk, case["scale"])
    torch.cuda.synchronize(dev)
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_decode(case, cache_np):
    return oracle.sparse_mla_decode(case["q"], cache_np, case["pt"], case["lens"], case["topk"],
                                    case["scale"])


def decode_plan(batch, heads, topk, fp8=False, tokens=1):
    """(workgroups sharing a list, splits, heads per group) of the library's
    plan, restated from its rule.
    Splits: as many as keep the busiest XCD (32 CUs; sequence s runs on XCD
    s % 8) at one workgroup per CU, at most 16, at most one per 64-row tile,
    and of at most 2048 (FP8: 1024) entries.  Head groups: 32 heads (16 at 16
    heads), or 16 at 64 heads where 32-head groups would leave splits of at
    most two tiles and 16-head groups give as many workgroups with more."""
    cap = 1024 if fp8 else 2048

    def splits(hg):
        s = max(1, 32 // (-(-batch // 8) * tokens * (heads // hg)))
        s = min(s, -(-topk // 64), 16)
        return max(s, -(-topk // cap))

    def tiles(s):
        return -(-(-(-topk // s)) // 64)

    hg = 32 if heads >= 32 else 16
    s = splits(hg)
    if heads == 64:
        s16 = splits(16)
        if tiles(s) <= 2 and tiles(s16) > tiles(s) and 4 * s16 >= 2 * s:
            hg, s = 16, s16
    return batch * tokens * (heads // hg), s, hg
