"""CPU pins of the oracle's storage-format code (E4M3, e2m1, row layout).

Each test fixes the oracle against something other than itself: PyTorch's
float8_e4m3fn (a library routine), brute force by exact distance over every
BF16 input, exact round trips, and the byte counts the pages print (kept in
tests/golden/page_figures.json with their citations).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])   # e2m1 magnitudes, by definition


def bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    return bits[finite]


def torch_e4m3_value(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_e4m3_encode(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def exact_ints(values, shift=160):
    """Dyadic doubles -> exact Python ints (value * 2**shift) in an object array.
    Every BF16 and E4M3 value is a multiple of 2**-133, so nothing is rounded."""
    out = []
    for v in np.asarray(values, dtype=np.float64).ravel():
        num, den = float(v).as_integer_ratio()
        out.append((num << shift) // den)
    return np.array(out, dtype=object)


def nearest_index_ties_even(dist):
    """Row-wise argmin of dist with ties going to the even column index."""
    m = dist.min(axis=1, keepdims=True)
    hit = dist == m
    n = dist.shape[1]
    even_first = np.concatenate([np.arange(0, n, 2), np.arange(1, n, 2)])
    cols = hit[:, even_first]
    first = cols.argmax(axis=1)
    # a tie between neighbours c, c+1 always contains exactly one even code
    return even_first[first]


# --------------------------------------------------------------------------
# E4M3
# --------------------------------------------------------------------------

def test_e4m3_table_matches_library():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_value(codes)
    ref = torch_e4m3_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])
    # spot values of the OCP E4M3FN definition
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0
    assert mine[0x08] == 2.0 ** -6 and mine[0x01] == 2.0 ** -9
    assert mine[0x80] == 0.0 and np.signbit(mine[0x80])


def test_e4m3_encode_inverts_decode():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    back = oracle.e4m3_nearest(oracle.e4m3_value(codes), 1.0)
    assert np.array_equal(back, codes)          # includes 0x80 (-0)


def test_e4m3_encode_all_bf16_against_library():
    bits = all_finite_bf16()
    x = bf16_bits_to_f64(bits)
    mine = oracle.e4m3_nearest(x, 1.0)
    inside = np.abs(x) <= 464.0                 # torch gives NaN past the last midpoint
    ref = torch_e4m3_encode(x[inside])
    assert np.array_equal(mine[inside], ref)
    sat = np.where(np.signbit(x[~inside]), 0xFE, 0x7E).astype(np.uint8)
    assert np.array_equal(mine[~inside], sat)


def test_e4m3_encode_brute_force_distance():
    """Nearest by exact distance over the whole finite grid, ties to even."""
    bits = all_finite_bf16()
    x = bf16_bits_to_f64(bits)
    grid = exact_ints(torch_e4m3_value(np.arange(0x7F, dtype=np.uint8)))   # 0x00..0x7E
    a = exact_ints(np.abs(x))
    code = np.empty(x.size, dtype=np.uint8)
    for lo in range(0, x.size, 4096):
        d = np.abs(a[lo:lo + 4096, None] - grid[None, :])
        code[lo:lo + 4096] = nearest_index_ties_even(d)
    code |= np.where(np.signbit(x), 0x80, 0).astype(np.uint8)
    assert np.array_equal(oracle.e4m3_nearest(x, 1.0), code)


# --------------------------------------------------------------------------
# block scale: nearest E4M3 to amax / 6
# --------------------------------------------------------------------------

def test_scale_rule_brute_force():
    bits = all_finite_bf16()
    amax = bf16_bits_to_f64(bits)
    amax = np.unique(np.abs(amax))
    grid6 = 6 * exact_ints(torch_e4m3_value(np.arange(0x7F, dtype=np.uint8)))
    a = exact_ints(amax)
    want = np.empty(amax.size, dtype=np.uint8)
    for lo in range(0, amax.size, 4096):
        d = np.abs(a[lo:lo + 4096, None] - grid6[None, :])
        want[lo:lo + 4096] = nearest_index_ties_even(d)
    got = oracle.e4m3_nearest(amax, 6.0)
    assert np.array_equal(got, want)
    # the same decisions through the library: fp32 divide, then torch's RNE cast
    inside = amax / 6.0 <= 464.0
    lib = torch_e4m3_encode((amax[inside].astype(np.float32) / np.float32(6.0)))
    assert np.array_equal(got[inside], lib)


# --------------------------------------------------------------------------
# e2m1
# --------------------------------------------------------------------------

def test_e2m1_table():
    nibs = np.arange(16, dtype=np.uint8)
    v = oracle.e2m1_value(nibs)
    assert np.array_equal(np.abs(v[:8]), E2M1) and np.array_equal(np.abs(v[8:]), E2M1)
    assert not np.signbit(v[:8]).any() and np.signbit(v[8:]).all()


def test_e2m1_encode_brute_force_every_scale():
    bits = all_finite_bf16()
    xall = bf16_bits_to_f64(bits)
    scales = torch_e4m3_value(np.arange(0x7F, dtype=np.uint8))
    checked = 0
    for S in scales:
        lim = 8.0 * S if S > 0 else 1.0
        x = xall[np.abs(xall) <= lim]
        got = oracle.e2m1_nearest(x, S)
        if S == 0:
            want = np.zeros(x.size, dtype=np.uint8)
        else:
            # an fp64 difference here can round only when |x| and S * g are far
            # apart, which is never next to a tie, so the argmin is exact
            d = np.abs(np.abs(x)[:, None] - S * E2M1[None, :])
            want = nearest_index_ties_even(d).astype(np.uint8)
        want |= np.where(np.signbit(x), 8, 0).astype(np.uint8)
        assert np.array_equal(got, want), S
        checked += x.size
    assert checked > 2_000_000


def _rocm_host_e2m1(tmpdir):
    """ROCm's software float -> e2m1 conversion (tests/hip_fp4_ref.cpp),
    built with hipcc, host code only; None without hipcc."""
    import ctypes
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        return None
    src = os.path.join(os.path.dirname(__file__), "hip_fp4_ref.cpp")
    so = os.path.join(str(tmpdir), "libhip_fp4_ref.so")
    r = subprocess.run([hipcc, "-std=c++17", "-O1", "-fPIC", "-shared", "-x", "hip", "--offload-host-only",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", src, "-o", so],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    lib = ctypes.CDLL(so)
    lib.hip_host_e2m1.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]

    def conv(x):
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.zeros(x.size, dtype=np.uint8)
        lib.hip_host_e2m1(x.ctypes.data, x.size, out.ctypes.data)
        return out
    return conv


def test_e2m1_encode_matches_rocm_host_reference(tmp_path):
    """The e2m1 rounding against a library routine: ROCm's software OCP FP4
    conversion (round to nearest even, saturating at 6) at block scale 1,
    and at power-of-two scales S, where x / S is exact.  Inputs: every
    multiple of 1/64 in [-10, 10] (all tie points among them), the floats
    next to each tie point, signed zeros, subnormals, saturating values and
    10^5 normal draws."""
    conv = _rocm_host_e2m1(tmp_path)
    if conv is None:
        pytest.skip("hipcc not found")
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    x = np.concatenate([
        np.arange(-640, 641, dtype=np.float32) / np.float32(64.0),
        np.array([0.0, -0.0, 1e-40, -1e-40, 6.0001, 5.9999, 1e30, -1e30], dtype=np.float32),
        np.nextafter(mids, np.float32(10.0)), np.nextafter(mids, np.float32(-10.0)),
        -np.nextafter(mids, np.float32(10.0)), -mids,
        np.random.default_rng(7).normal(0.0, 3.0, 100_000).astype(np.float32)])
    want = conv(x)
    assert np.array_equal(oracle.e2m1_nearest(x.astype(np.float64), 1.0), want)
    for k in (-6, -2, 3, 8):
        S = 2.0 ** k
        assert np.array_equal(oracle.e2m1_nearest(x.astype(np.float64) * S, S), want), k


def test_e2m1_tie_points():
    S = 1.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    # ties go to the even code: 0, 2, 2, 4, 4, 6, 6
    assert list(oracle.e2m1_nearest(mids, S)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.e2m1_nearest(np.array([7.0, 100.0, -100.0]), S)) == [7, 7, 15]


# --------------------------------------------------------------------------
# rows
# --------------------------------------------------------------------------

def _f64_to_bf16_exact(v):
    f = np.asarray(v, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), v)
    u = f.view(np.uint32)
    assert not (u & 0xFFFF).any(), "value not representable in bf16"
    return (u >> 16).astype(np.uint16)


def _independent_decode(rows):
    """Row bytes -> values, via torch's E4M3 and the e2m1 magnitude table."""
    rows = np.asarray(rows, dtype=np.uint8)
    nib = np.empty((rows.shape[0], 512), dtype=np.uint8)
    nib[:, 0::2] = rows[:, :256] & 0xF
    nib[:, 1::2] = rows[:, :256] >> 4
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0)
    S = torch_e4m3_value(rows[:, 256:288])
    lat = mag * np.repeat(S, 16, axis=1)
    rope = torch_e4m3_value(rows[:, 288:352])
    return np.concatenate([lat, rope], axis=1)


def test_row_round_trip_every_scale():
    rng = np.random.default_rng(11)
    scales = np.arange(1, 0x7F, dtype=np.uint8)            # every positive finite scale
    n = scales.size * 4
    rows = np.zeros((n, 352), dtype=np.uint8)
    nib = rng.integers(0, 16, size=(n, 512)).astype(np.uint8)
    # force one +-6 per block so that amax = 6 * S exactly
    pos = rng.integers(0, 16, size=(n, 32))
    sign = rng.integers(0, 2, size=(n, 32)).astype(np.uint8) * 8
    for blk in range(32):
        nib[np.arange(n), blk * 16 + pos[:, blk]] = 7 | sign[:, blk]
    rows[:, :256] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    sc = np.tile(scales, 4)
    rows[:, 256:288] = rng.choice(scales, size=(n, 32))
    rows[:, 256] = sc                                        # every scale appears
    rope = rng.integers(0, 256, size=(n, 64)).astype(np.uint8)
    rope[(rope & 0x7F) == 0x7F] = 0x7E
    rows[:, 288:] = rope
    vals = oracle.dequant_rows(rows)
    assert np.array_equal(vals, _independent_decode(rows))
    back = oracle.quant_rows(_f64_to_bf16_exact(vals))
    # a -0 nibble decodes to -0.0 and re-encodes to 0x8; everything is bit-exact
    assert np.array_equal(back, rows)


def test_row_layout_single_nonzero():
    one = np.uint16(0x3F80)                                  # bf16 1.0
    for d in list(range(0, 512, 37)) + [1, 510, 511]:
        x = np.zeros((1, 576), dtype=np.uint16)
        x[0, d] = one
        row = oracle.quant_rows(x)[0]
        want = np.zeros(352, dtype=np.uint8)
        # scale: E4M3 nearest 1/6 is 0.171875 = 1.375 * 2^-3 -> e=4, m=3 -> 0x23;
        # 1 / 0.171875 = 5.82 -> e2m1 6.0 (code 7)
        want[256 + d // 16] = 0x23
        want[d // 2] = 7 if d % 2 == 0 else 0x70
        assert np.array_equal(row, want), d
    for j in (0, 17, 63):
        x = np.zeros((1, 576), dtype=np.uint16)
        x[0, 512 + j] = one
        row = oracle.quant_rows(x)[0]
        want = np.zeros(352, dtype=np.uint8)
        want[288 + j] = 0x38
        assert np.array_equal(row, want), j


def test_row_special_blocks():
    x = np.zeros((5, 576), dtype=np.uint16)
    x[1, :16] = 0x8000                                       # all -0
    x[2, :16] = _f64_to_bf16_exact(np.full(16, 6.0 * 2.0 ** -10))       # tie with 0 -> 0
    x[3, :16] = _f64_to_bf16_exact(np.full(16, 6.0 * 2.0 ** -10)) + 1   # next bf16 above
    x[4, :16] = _f64_to_bf16_exact(np.full(16, 4096.0))     # saturating scale
    r = oracle.quant_rows(x)
    assert not r[0].any()
    assert (r[1, :8] == 0x88).all() and r[1, 256] == 0 and not r[1, 8:].any()
    assert r[2, 256] == 0x00 and not r[2, :8].any()
    assert r[3, 256] == 0x01
    assert r[4, 256] == 0x7E and (r[4, :8] == 0x77).all()
    vals = oracle.dequant_rows(r)
    assert not vals[2].any()


def test_layout_constants_match_pages():
    g = json.load(open(GOLDEN))
    rb = g["row_bytes"]
    assert rb["nvfp4_row"]["latent"] == rb["latent_values"] // 2
    assert rb["nvfp4_row"]["scales"] == rb["latent_values"] // rb["values_per_scale"]
    assert rb["nvfp4_row"]["rope"] == rb["rope_values"]
    total = rb["nvfp4_row"]["latent"] + rb["nvfp4_row"]["scales"] + rb["nvfp4_row"]["rope"]
    assert total == rb["nvfp4_row"]["total"] == 352
    assert oracle.quant_rows(np.zeros((1, 576), np.uint16)).shape == (1, total)
    assert oracle._load().oracle_row_bytes() == total
    assert oracle._load().oracle_page_rows() == g["page_tokens"]["tokens"]
    ls = g["latent_share"]
    assert 100.0 * (rb["nvfp4_row"]["latent"] + rb["nvfp4_row"]["scales"]) / ls["fp8_latent"] \
        == ls["percent"]
    assert round(rb["fp8_row"]["total"] / total, 2) == g["per_row_ratio"]["ratio_2dp"]
    st = g["staged_bytes_per_row"]
    assert sum(st["parts"]) == st["staged"] and st["parts"][0] == total
    assert round(st["staged"] / total, 1) == st["ratio_1dp"]
    sb = g["session_bytes"]
    assert round(sb["tokens"] * sb["layers"] * rb["fp8_row"]["total"] / 1e9, 1) == sb["fp8_GB_1dp"]
    assert round(sb["tokens"] * sb["layers"] * total / 1e9, 1) == sb["nvfp4_GB_1dp"]
    rq = g["request_bytes"]
    assert round(rq["tokens"] * rq["layers"] * total / 1e9, 1) == rq["nvfp4_GB_1dp"]


def test_append_slot_rules():
    """The paged append writes row i to slot s = page * 64 + row and skips a
    slot outside [0, num_pages * 64): -1, -2^31, num_pages * 64 and 2^31 - 1.
    The cache is a window of a larger array, so a row written just outside it
    lands in a guard band that must stay untouched."""
    P = 2
    backing = np.full((P + 4, 64, 352), 0xAB, dtype=np.uint8)
    cache = backing[2:2 + P]
    assert cache.flags.c_contiguous
    g = torch.Generator().manual_seed(31)
    x = wl.bf16_bits(torch.randn((5, 576), generator=g).to(torch.bfloat16))
    slots = np.array([5, -1, P * 64, 127, 64], dtype=np.int32)
    assert oracle.kv_quant_append(x, slots, cache) == 3
    rows = oracle.quant_rows(x)
    flat = backing.reshape(-1, 352)
    base = 2 * 64
    want = np.full_like(flat, 0xAB)
    want[base + 5], want[base + 127], want[base + 64] = rows[0], rows[3], rows[4]
    assert np.array_equal(flat, want)
    # the extreme int32 slots are skipped too (nothing written, nothing read)
    far = np.array([-2 ** 31, 2 ** 31 - 1, 0], dtype=np.int32)
    assert oracle.kv_quant_append(x[:3], far, cache) == 1
    want[base + 0] = rows[2]
    assert np.array_equal(flat, want)
