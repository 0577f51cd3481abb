"""CPU oracle for sparse NVFP4-MLA decode -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library in
``sparse_mla_decode_amd`` never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, fp64, scalar loops); this
module only builds it with gcc and marshals numpy arrays through ctypes.
BF16 tensors travel as their uint16 bit patterns (numpy has no bfloat16).

Every function here is pinned by the CPU tests in ``tests/test_oracle_*.py``
(exhaustive format tables against PyTorch's float8_e4m3fn, brute force over
all BF16 inputs, dense attention through a library routine, one-hot, uniform
and single-entry closed forms, invariances, and the byte counts the pages
print, stored under ``tests/golden/``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# SMLA_ORACLE_SANITIZE=1 selects a second build of the same source with
# AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload
# their runtimes; tests/test_oracle_sanitize.py does this).
_SANITIZE = os.environ.get("SMLA_ORACLE_SANITIZE") == "1"
_LIB = os.path.join(_HERE, "liboracle_san.so" if _SANITIZE else "liboracle.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"]

ROW_BYTES = 352
FP8_ROW_BYTES = 576
PAGE_ROWS = 64
LATENT = 512
DIM = 576

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-std=c11", "-Wall", *(_SAN_FLAGS if _SANITIZE else []),
               "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64, i32, u8, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint8, ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [u8]
    lib.oracle_e4m3_value.restype = dbl
    lib.oracle_e4m3_nearest.argtypes = [dbl, dbl]
    lib.oracle_e4m3_nearest.restype = u8
    lib.oracle_e2m1_value.argtypes = [u8]
    lib.oracle_e2m1_value.restype = dbl
    lib.oracle_e2m1_nearest.argtypes = [dbl, dbl]
    lib.oracle_e2m1_nearest.restype = u8
    lib.oracle_e4m3_value_many.argtypes = [P, i64, P]
    lib.oracle_e4m3_value_many.restype = None
    lib.oracle_e4m3_nearest_many.argtypes = [P, i64, dbl, P]
    lib.oracle_e4m3_nearest_many.restype = None
    lib.oracle_e2m1_nearest_many.argtypes = [P, P, i64, P]
    lib.oracle_e2m1_nearest_many.restype = None
    lib.oracle_quant_rows.argtypes = [P, i64, P]
    lib.oracle_quant_rows.restype = None
    lib.oracle_dequant_rows.argtypes = [P, i64, P]
    lib.oracle_dequant_rows.restype = None
    lib.oracle_kv_quant_append.argtypes = [P, i64, P, P, i64]
    lib.oracle_kv_quant_append.restype = i64
    lib.oracle_sparse_mla_decode.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, dbl,
                                             P, P, ctypes.c_int]
    lib.oracle_sparse_mla_decode.restype = None
    lib.oracle_quant_rows_fp8.argtypes = [P, i64, P]
    lib.oracle_quant_rows_fp8.restype = None
    lib.oracle_dequant_rows_fp8.argtypes = [P, i64, P]
    lib.oracle_dequant_rows_fp8.restype = None
    lib.oracle_kv_quant_append_fp8.argtypes = [P, i64, P, P, i64]
    lib.oracle_kv_quant_append_fp8.restype = i64
    lib.oracle_sparse_mla_decode_fp8.argtypes = lib.oracle_sparse_mla_decode.argtypes
    lib.oracle_sparse_mla_decode_fp8.restype = None
    lib.oracle_stage_rows_fp8.argtypes = [P, i64, P, i32, P, P, i32, i32, P, P]
    lib.oracle_stage_rows_fp8.restype = None
    lib.oracle_topk_select.argtypes = [P, i64, P, i32, i32, P]
    lib.oracle_topk_select.restype = None
    lib.oracle_fp8_row_bytes.restype = ctypes.c_int
    lib.oracle_row_bytes.restype = ctypes.c_int
    lib.oracle_page_rows.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# -- format functions, vectorised over numpy arrays ------------------------

def e4m3_value(codes) -> np.ndarray:
    """Exact value of each E4M3FN code (NaN for S.1111.111)."""
    c = _c(codes, np.uint8)
    out = np.zeros(c.shape, dtype=np.float64)
    _load().oracle_e4m3_value_many(_ptr(c), c.size, _ptr(out))
    return out


def e4m3_nearest(num, den: float = 1.0) -> np.ndarray:
    """Code of the E4M3 value nearest num/den (ties to even, saturating)."""
    x = _c(num, np.float64)
    out = np.zeros(x.shape, dtype=np.uint8)
    _load().oracle_e4m3_nearest_many(_ptr(x), x.size, float(den), _ptr(out))
    return out


def e2m1_value(nibs) -> np.ndarray:
    lib = _load()
    nibs = np.asarray(nibs, dtype=np.uint8)
    return np.array([lib.oracle_e2m1_value(int(c)) for c in nibs.ravel()],
                    dtype=np.float64).reshape(nibs.shape)


def e2m1_nearest(x, S) -> np.ndarray:
    """Nibble nearest x / S (ties to even code, saturating, sign copied)."""
    xx = _c(x, np.float64)
    SS = _c(np.broadcast_to(np.asarray(S, dtype=np.float64), xx.shape), np.float64)
    out = np.zeros(xx.shape, dtype=np.uint8)
    _load().oracle_e2m1_nearest_many(_ptr(xx), _ptr(SS), xx.size, _ptr(out))
    return out


# -- rows ---------------------------------------------------------------

def set_threads(nthreads: int) -> int:
    """Thread count of the row quantisers' OpenMP loops for later calls from
    this thread (timing only; the results do not depend on it).  Returns the
    count they will use."""
    return int(_load().oracle_set_threads(int(nthreads)))


def quant_rows(rows_bf16_bits: np.ndarray) -> np.ndarray:
    """[n,576] uint16 (BF16 bit patterns) -> [n,352] uint8 NVFP4 rows."""
    x = _c(rows_bf16_bits, np.uint16)
    assert x.ndim == 2 and x.shape[1] == DIM, x.shape
    out = np.zeros((x.shape[0], ROW_BYTES), dtype=np.uint8)
    if x.shape[0]:
        _load().oracle_quant_rows(_ptr(x), x.shape[0], _ptr(out))
    return out


def dequant_rows(rows: np.ndarray) -> np.ndarray:
    """[n,352] uint8 -> [n,576] float64 exact values."""
    r = _c(rows, np.uint8)
    assert r.ndim == 2 and r.shape[1] == ROW_BYTES, r.shape
    out = np.zeros((r.shape[0], DIM), dtype=np.float64)
    if r.shape[0]:
        _load().oracle_dequant_rows(_ptr(r), r.shape[0], _ptr(out))
    return out


def kv_quant_append(rows_bf16_bits: np.ndarray, slot_mapping: np.ndarray,
                    cache: np.ndarray) -> int:
    """Quantise rows into ``cache`` ([P,64,352] uint8, modified in place)."""
    x = _c(rows_bf16_bits, np.uint16)
    s = _c(slot_mapping, np.int32)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous
    assert cache.ndim == 3 and cache.shape[1:] == (PAGE_ROWS, ROW_BYTES)
    assert x.shape == (s.shape[0], DIM)
    return int(_load().oracle_kv_quant_append(_ptr(x), x.shape[0], _ptr(s), _ptr(cache),
                                              cache.shape[0]))


def quant_rows_fp8(rows_bf16_bits: np.ndarray) -> np.ndarray:
    """[n,576] uint16 (BF16 bit patterns) -> [n,576] uint8 lean FP8 rows."""
    x = _c(rows_bf16_bits, np.uint16)
    assert x.ndim == 2 and x.shape[1] == DIM, x.shape
    out = np.zeros((x.shape[0], FP8_ROW_BYTES), dtype=np.uint8)
    if x.shape[0]:
        _load().oracle_quant_rows_fp8(_ptr(x), x.shape[0], _ptr(out))
    return out


def dequant_rows_fp8(rows: np.ndarray) -> np.ndarray:
    """[n,576] uint8 lean FP8 rows -> [n,576] float64 exact values."""
    r = _c(rows, np.uint8)
    assert r.ndim == 2 and r.shape[1] == FP8_ROW_BYTES, r.shape
    out = np.zeros((r.shape[0], DIM), dtype=np.float64)
    if r.shape[0]:
        _load().oracle_dequant_rows_fp8(_ptr(r), r.shape[0], _ptr(out))
    return out


def kv_quant_append_fp8(rows_bf16_bits: np.ndarray, slot_mapping: np.ndarray,
                        cache: np.ndarray) -> int:
    """Quantise rows into the lean FP8 ``cache`` ([P,64,576] uint8, in place)."""
    x = _c(rows_bf16_bits, np.uint16)
    s = _c(slot_mapping, np.int32)
    assert cache.dtype == np.uint8 and cache.flags.c_contiguous
    assert cache.ndim == 3 and cache.shape[1:] == (PAGE_ROWS, FP8_ROW_BYTES)
    assert x.shape == (s.shape[0], DIM)
    return int(_load().oracle_kv_quant_append_fp8(_ptr(x), x.shape[0], _ptr(s), _ptr(cache),
                                                  cache.shape[0]))


def stage_rows_fp8(cache: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray,
                   topk: np.ndarray, staged: np.ndarray | None = None):
    """The staged path's gather-unpack: returns (staged [B*kpad/64, 64, 576]
    lean FP8 rows, staged_topk [B, K]); entry e of sequence b goes to row
    b*kpad + e (kpad = K rounded up to 64), staged_topk = e or -1.  Rows of
    unusable entries keep the contents of `staged` (zeros if not given)."""
    c = _c(cache, np.uint8)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    tk = _c(topk, np.int32)
    assert c.ndim == 3 and c.shape[1:] == (PAGE_ROWS, ROW_BYTES)
    B, K = tk.shape
    kpad = -(-K // PAGE_ROWS) * PAGE_ROWS
    if staged is None:
        staged = np.zeros((B * kpad // PAGE_ROWS, PAGE_ROWS, FP8_ROW_BYTES), dtype=np.uint8)
    assert staged.dtype == np.uint8 and staged.flags.c_contiguous
    assert staged.shape == (B * kpad // PAGE_ROWS, PAGE_ROWS, FP8_ROW_BYTES)
    st = np.zeros((B, K), dtype=np.int32)
    _load().oracle_stage_rows_fp8(_ptr(c), c.shape[0], _ptr(pt), pt.shape[1], _ptr(sl), _ptr(tk),
                                  B, K, _ptr(staged), _ptr(st))
    return staged, st


def staged_tables(batch: int, topk_len: int):
    """Page table and seq_lens of the staged copy: page [b][p] = b*kpad/64 + p."""
    pp = -(-topk_len // PAGE_ROWS)
    pt = np.arange(batch * pp, dtype=np.int32).reshape(batch, pp)
    return pt, np.full(batch, pp * PAGE_ROWS, dtype=np.int32)


def sparse_mla_decode_mtp(q_bf16_bits: np.ndarray, cache: np.ndarray, page_table: np.ndarray,
                          seq_lens: np.ndarray, topk: np.ndarray, softmax_scale: float,
                          nthreads: int = 0):
    """Multi-token decode ("GLM-5.3 PCP/DCP long-context on H200", section 4:
    MTP speculative decoding with draft tokens): q [B,T,H,576] BF16 bits,
    topk [B,T,K], page table and seq_lens per sequence.  Token j of sequence
    b sits at position L_b - T + j and attends over its own list, whose
    usable entries are those of the decode with length L_b - (T - 1 - j).
    Returns (out [B,T,H,512], lse [B,T,H]) in fp64."""
    q = _c(q_bf16_bits, np.uint16)
    B, T, H, D = q.shape
    tk = _c(topk, np.int32)
    assert tk.shape[:2] == (B, T)
    pt = np.repeat(_c(page_table, np.int32), T, axis=0)
    lens = np.asarray(seq_lens, dtype=np.int64)
    lens_q = (lens[:, None] - (T - 1 - np.arange(T))[None, :]).reshape(-1)
    out, lse = sparse_mla_decode(q.reshape(B * T, H, D), cache, pt, lens_q,
                                 tk.reshape(B * T, -1), softmax_scale, nthreads)
    return out.reshape(B, T, H, -1), lse.reshape(B, T, H)


def topk_select(scores: np.ndarray, seq_lens: np.ndarray, topk: int) -> np.ndarray:
    """[B, ld] float32 scores -> [B, topk] int32: the positions of the
    min(topk, L_b) largest scores of row b (L_b = seq_lens[b] clamped to
    [0, ld]), best first, equal scores by lower position, then -1."""
    x = _c(scores, np.float32)
    sl = _c(seq_lens, np.int32)
    assert x.ndim == 2 and sl.shape == (x.shape[0],)
    out = np.zeros((x.shape[0], topk), dtype=np.int32)
    _load().oracle_topk_select(_ptr(x), x.shape[1], _ptr(sl), x.shape[0], int(topk), _ptr(out))
    return out


def sparse_mla_decode(q_bf16_bits: np.ndarray, cache: np.ndarray, page_table: np.ndarray,
                      seq_lens: np.ndarray, topk: np.ndarray, softmax_scale: float,
                      nthreads: int = 0):
    """Returns (out [B,H,512] float64, lse [B,H] float64).  The cache's row
    size selects the format: [P,64,352] NVFP4 rows or [P,64,576] lean FP8
    rows."""
    q = _c(q_bf16_bits, np.uint16)
    c = _c(cache, np.uint8)
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    tk = _c(topk, np.int32)
    B, H, D = q.shape
    assert D == DIM and c.ndim == 3 and c.shape[1] == PAGE_ROWS
    assert c.shape[2] in (ROW_BYTES, FP8_ROW_BYTES), c.shape
    assert pt.ndim == 2 and pt.shape[0] == B and sl.shape == (B,)
    assert tk.ndim == 2 and tk.shape[0] == B
    out = np.zeros((B, H, LATENT), dtype=np.float64)
    lse = np.zeros((B, H), dtype=np.float64)
    lib = _load()
    fn = lib.oracle_sparse_mla_decode if c.shape[2] == ROW_BYTES else lib.oracle_sparse_mla_decode_fp8
    fn(_ptr(q), _ptr(c), c.shape[0], _ptr(pt), pt.shape[1], _ptr(sl), _ptr(tk), B, H, tk.shape[1],
       float(softmax_scale), _ptr(out), _ptr(lse), int(nthreads))
    return out, lse
