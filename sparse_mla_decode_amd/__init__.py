"""Sparse NVFP4-MLA decode on MI355X (gfx950): Python binding of libsmla.so.

This module is argument marshalling only.  Every step of the path runs in the
HIP kernels behind the C ABI in ``include/smla.h``; PyTorch provides device
memory and the current stream.  There is no fallback: if ``libsmla.so`` has
not been built, importing this package raises.

    kv_quant_append(rows, slot_mapping, cache)
        rows [n,576] bf16, slot_mapping [n] int32, cache [P,64,352] uint8 (in place)
    sparse_mla_decode(q, cache, page_table, seq_lens, topk, softmax_scale)
        -> (out [B,H,512] fp32, lse [B,H] fp32)
    append_decode(new_rows [B,576] bf16, new_slots [B] int32, q, cache, ...)
        kv_quant_append of each sequence's newest row, then the decode, in one
        launch (the same cache bytes, out and lse)
    kv_quant_append_fp8, sparse_mla_decode_fp8
        the same over the lean FP8 row: cache [P,64,576] uint8
    stage_rows_fp8, sparse_mla_decode_staged
        the staged path (NVFP4 rows -> FP8 copy in HBM -> FP8 decode), kept
        to measure the fused kernel against
    sparse_mla_decode_mtp(q [B,T,H,576], cache, page_table, seq_lens, topk [B,T,K], scale)
        T query tokens per sequence (MTP drafts), each with its own list
    topk_select(scores, seq_lens, topk) -> topk [B,K] int32
        the positions of each query's K largest scores (the decode's list)
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsmla.so")

LATENT = 512
ROPE = 64
DIM = 576
ROW_BYTES = 352
FP8_ROW_BYTES = 576
PAGE_ROWS = 64
MAX_TOPK = 2048

ERRORS = {
    0: "SMLA_OK", -1: "SMLA_ERR_NULL", -2: "SMLA_ERR_SHAPE", -3: "SMLA_ERR_UNSUPPORTED",
    -4: "SMLA_ERR_ALIGN", -5: "SMLA_ERR_WORKSPACE", -6: "SMLA_ERR_LAUNCH", -7: "SMLA_ERR_DEVICE",
    -8: "SMLA_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 << 20   # SMLA_NOALLOC_SCRATCH_BYTES

# exported symbols, in the order include/smla.h declares them
EXPORTS = ("smla_strerror", "smla_version", "smla_kv_quant_append",
           "smla_decode_workspace_bytes", "smla_sparse_mla_decode", "smla_kv_quant_append_fp8",
           "smla_decode_workspace_bytes_fp8", "smla_sparse_mla_decode_fp8",
           "smla_stage_rows_fp8", "smla_decode_workspace_bytes_mtp", "smla_sparse_mla_decode_mtp",
           "smla_topk_workspace_bytes", "smla_topk_select", "smla_sparse_mla_decode_noalloc",
           "smla_append_decode")


class SmlaError(RuntimeError):
    def __init__(self, code: int, lib):
        msg = lib.smla_strerror(code).decode()
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libsmla.so is not built (expected %s); run `python -c \"import "
            "__graft_entry__ as g; g.build()\"` or `python sparse_mla_decode_amd/build.py`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, f32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                            ctypes.c_size_t)
    lib.smla_strerror.argtypes = [ctypes.c_int]
    lib.smla_strerror.restype = ctypes.c_char_p
    lib.smla_version.argtypes = []
    lib.smla_version.restype = ctypes.c_int
    for sfx in ("", "_fp8"):
        fn = getattr(lib, "smla_kv_quant_append" + sfx)
        fn.argtypes = [P, i64, P, P, i64, P]
        fn.restype = ctypes.c_int
        fn = getattr(lib, "smla_decode_workspace_bytes" + sfx)
        fn.argtypes = [i32, i32, i32]
        fn.restype = sz
        fn = getattr(lib, "smla_sparse_mla_decode" + sfx)
        fn.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, f32, P, P, P, sz, P]
        fn.restype = ctypes.c_int
    lib.smla_stage_rows_fp8.argtypes = [P, i64, P, i32, P, P, i32, i32, P, P, P]
    lib.smla_stage_rows_fp8.restype = ctypes.c_int
    lib.smla_decode_workspace_bytes_mtp.argtypes = [i32, i32, i32, i32]
    lib.smla_decode_workspace_bytes_mtp.restype = sz
    lib.smla_sparse_mla_decode_mtp.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, i32, f32,
                                               P, P, P, sz, P]
    lib.smla_sparse_mla_decode_mtp.restype = ctypes.c_int
    lib.smla_topk_workspace_bytes.argtypes = [i32, i64]
    lib.smla_topk_workspace_bytes.restype = sz
    lib.smla_topk_select.argtypes = [P, i64, P, i32, i32, P, P, sz, P]
    lib.smla_topk_select.restype = ctypes.c_int
    lib.smla_sparse_mla_decode_noalloc.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, f32, P,
                                                   P, P]
    lib.smla_sparse_mla_decode_noalloc.restype = ctypes.c_int
    lib.smla_append_decode.argtypes = [P, P, P, P, i64, P, i32, P, P, i32, i32, i32, f32, P, P, P,
                                       sz, P]
    lib.smla_append_decode.restype = ctypes.c_int
    return lib


lib = _load()

_ws_lock = threading.Lock()
_workspaces: dict = {}


def _check(code: int):
    if code != 0:
        raise SmlaError(code, lib)


# torch's raw current-stream query: the same pointer as
# torch.cuda.current_stream(device).cuda_stream without building a Stream
# object (0.07 us against 2 us per call, a large share of a call's host time)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_ptr(device: torch.device, stream=None) -> int:
    if stream is None:
        if _raw_stream is not None and device.index is not None:
            return int(_raw_stream(device.index))
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _req(t: torch.Tensor, name: str, dtype, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_cuda:
        raise ValueError("%s must be on a GPU" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _req_shape(t: torch.Tensor, name: str, dtype, shape: tuple, device):
    _req(t, name, dtype, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _req_workspace(ws, device) -> tuple:
    """(pointer, bytes) of a caller-supplied workspace: a contiguous tensor
    on the call's device (any dtype), or (None, 0)."""
    if ws is None:
        return None, 0
    if not isinstance(ws, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if not ws.is_cuda or ws.device != device:
        raise ValueError("workspace is on %s, expected %s" % (ws.device, device))
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.data_ptr(), ws.numel() * ws.element_size()


def version() -> int:
    return int(lib.smla_version())


def decode_workspace_bytes(batch: int, heads: int, topk: int) -> int:
    return int(lib.smla_decode_workspace_bytes(batch, heads, topk))


def decode_workspace_bytes_fp8(batch: int, heads: int, topk: int) -> int:
    return int(lib.smla_decode_workspace_bytes_fp8(batch, heads, topk))


def workspace_for(device: torch.device, nbytes: int, stream=None) -> torch.Tensor:
    """A workspace of at least nbytes, cached per (device, stream)."""
    key = (device.index, _stream_ptr(device, stream))
    with _ws_lock:
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            _workspaces[key] = ws
        return ws


def _append(rows, slot_mapping, cache, stream, row_bytes, fn):
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(rows, "rows", torch.bfloat16, 2, dev)
    _req(slot_mapping, "slot_mapping", torch.int32, 1, dev)
    if rows.shape[1] != DIM or slot_mapping.shape[0] != rows.shape[0]:
        raise ValueError("rows must be [n,576] and slot_mapping [n]")
    if tuple(cache.shape[1:]) != (PAGE_ROWS, row_bytes):
        raise ValueError("cache must be [num_pages,64,%d]" % row_bytes)
    _check(fn(rows.data_ptr(), rows.shape[0], slot_mapping.data_ptr(), cache.data_ptr(),
              cache.shape[0], _stream_ptr(dev, stream)))


def kv_quant_append(rows: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                    stream=None) -> None:
    """Quantise BF16 rows [n,576] into cache slots (page*64 + row) of cache [P,64,352]."""
    _append(rows, slot_mapping, cache, stream, ROW_BYTES, lib.smla_kv_quant_append)


def kv_quant_append_fp8(rows: torch.Tensor, slot_mapping: torch.Tensor, cache: torch.Tensor,
                        stream=None) -> None:
    """Quantise BF16 rows [n,576] into lean FP8 rows of cache [P,64,576]."""
    _append(rows, slot_mapping, cache, stream, FP8_ROW_BYTES, lib.smla_kv_quant_append_fp8)


def _decode(q, cache, page_table, seq_lens, topk, softmax_scale, out, lse, workspace, stream,
            row_bytes, fn, ws_fn, prefix=()):
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(q, "q", torch.bfloat16, 3, dev)
    _req(page_table, "page_table", torch.int32, 2, dev)
    _req(seq_lens, "seq_lens", torch.int32, 1, dev)
    _req(topk, "topk", torch.int32, 2, dev)
    B, H, D = q.shape
    if D != DIM:
        raise ValueError("q must be [B,H,576]")
    if tuple(cache.shape[1:]) != (PAGE_ROWS, row_bytes):
        raise ValueError("cache must be [num_pages,64,%d]" % row_bytes)
    if page_table.shape[0] != B or seq_lens.shape[0] != B or topk.shape[0] != B:
        raise ValueError("page_table, seq_lens and topk need one row per sequence")
    K = topk.shape[1]
    if out is None:
        out = torch.empty((B, H, LATENT), dtype=torch.float32, device=dev)
    else:
        _req_shape(out, "out", torch.float32, (B, H, LATENT), dev)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    else:
        _req_shape(lse, "lse", torch.float32, (B, H), dev)
    need = int(ws_fn(B, H, K))
    if workspace is None and need > 0:
        workspace = workspace_for(dev, need, stream)
    ws_ptr, ws_bytes = _req_workspace(workspace, dev)
    _check(fn(*prefix, q.data_ptr(), cache.data_ptr(), cache.shape[0], page_table.data_ptr(),
              page_table.shape[1], seq_lens.data_ptr(), topk.data_ptr(), B, H, K,
              float(softmax_scale), out.data_ptr(), lse.data_ptr(), ws_ptr, ws_bytes,
              _stream_ptr(dev, stream)))
    return out, lse


def sparse_mla_decode(q: torch.Tensor, cache: torch.Tensor, page_table: torch.Tensor,
                      seq_lens: torch.Tensor, topk: torch.Tensor, softmax_scale: float,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None, stream=None):
    """Sparse MLA decode over cache [P,64,352]; returns (out [B,H,512] fp32, lse [B,H] fp32)."""
    return _decode(q, cache, page_table, seq_lens, topk, softmax_scale, out, lse, workspace,
                   stream, ROW_BYTES, lib.smla_sparse_mla_decode, lib.smla_decode_workspace_bytes)


def append_decode(new_rows: torch.Tensor, new_slots: torch.Tensor, q: torch.Tensor,
                  cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                  topk: torch.Tensor, softmax_scale: float, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                  stream=None):
    """kv_quant_append(new_rows [B,576] bf16, new_slots [B] int32, cache), then
    sparse_mla_decode(q, cache, ...), in one launch: returns (out, lse).  The
    slots must be distinct and each read by its own sequence's list alone."""
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(q, "q", torch.bfloat16, 3, dev)
    _req(new_rows, "new_rows", torch.bfloat16, 2, dev)
    _req(new_slots, "new_slots", torch.int32, 1, dev)
    if tuple(new_rows.shape) != (q.shape[0], DIM) or new_slots.shape[0] != q.shape[0]:
        raise ValueError("new_rows must be [B,576] and new_slots [B]")
    return _decode(q, cache, page_table, seq_lens, topk, softmax_scale, out, lse, workspace,
                   stream, ROW_BYTES, lib.smla_append_decode, lib.smla_decode_workspace_bytes,
                   prefix=(new_rows.data_ptr(), new_slots.data_ptr()))


def sparse_mla_decode_noalloc(q: torch.Tensor, cache: torch.Tensor, page_table: torch.Tensor,
                              seq_lens: torch.Tensor, topk: torch.Tensor, softmax_scale: float,
                              out: torch.Tensor, lse: torch.Tensor, stream=None):
    """sparse_mla_decode through the entry point that allocates nothing: the
    caller passes out [B,H,512] and lse [B,H]; the split partials use the
    library's static scratch (calls overlapping on one GPU race on it)."""
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(q, "q", torch.bfloat16, 3, dev)
    _req(page_table, "page_table", torch.int32, 2, dev)
    _req(seq_lens, "seq_lens", torch.int32, 1, dev)
    _req(topk, "topk", torch.int32, 2, dev)
    B, H, D = q.shape
    if D != DIM or tuple(cache.shape[1:]) != (PAGE_ROWS, ROW_BYTES):
        raise ValueError("q must be [B,H,576] and cache [num_pages,64,352]")
    if page_table.shape[0] != B or seq_lens.shape[0] != B or topk.shape[0] != B:
        raise ValueError("page_table, seq_lens and topk need one row per sequence")
    _req_shape(out, "out", torch.float32, (B, H, LATENT), dev)
    _req_shape(lse, "lse", torch.float32, (B, H), dev)
    _check(lib.smla_sparse_mla_decode_noalloc(
        q.data_ptr(), cache.data_ptr(), cache.shape[0], page_table.data_ptr(), page_table.shape[1],
        seq_lens.data_ptr(), topk.data_ptr(), B, H, topk.shape[1], float(softmax_scale),
        out.data_ptr(), lse.data_ptr(), _stream_ptr(dev, stream)))
    return out, lse


def sparse_mla_decode_fp8(q: torch.Tensor, cache: torch.Tensor, page_table: torch.Tensor,
                          seq_lens: torch.Tensor, topk: torch.Tensor, softmax_scale: float,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None):
    """The same decode over the lean FP8 cache [P,64,576]."""
    return _decode(q, cache, page_table, seq_lens, topk, softmax_scale, out, lse, workspace,
                   stream, FP8_ROW_BYTES, lib.smla_sparse_mla_decode_fp8,
                   lib.smla_decode_workspace_bytes_fp8)


_staged_tables: dict = {}


def staged_tables(batch: int, topk: int, device: torch.device):
    """Page table [batch][kpad/64] (b*kpad/64 + p) and seq_lens (all kpad) of
    the staged copy, cached per (device, batch, topk)."""
    key = (device.index, batch, topk)
    with _ws_lock:
        t = _staged_tables.get(key)
        if t is None:
            pp = (topk + PAGE_ROWS - 1) // PAGE_ROWS
            pt = torch.arange(batch * pp, dtype=torch.int32, device=device).view(batch, pp)
            sl = torch.full((batch,), pp * PAGE_ROWS, dtype=torch.int32, device=device)
            t = _staged_tables[key] = (pt, sl)
        return t



def stage_rows_fp8(cache: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                   topk: torch.Tensor, staged: torch.Tensor | None = None,
                   staged_topk: torch.Tensor | None = None, stream=None):
    """The staged path's gather-unpack: NVFP4 rows of the usable entries ->
    lean FP8 copy [B*kpad/64, 64, 576] (entry e of sequence b at row b*kpad+e)
    and staged_topk [B, K] (e or -1).  Returns (staged, staged_topk)."""
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(page_table, "page_table", torch.int32, 2, dev)
    _req(seq_lens, "seq_lens", torch.int32, 1, dev)
    _req(topk, "topk", torch.int32, 2, dev)
    if tuple(cache.shape[1:]) != (PAGE_ROWS, ROW_BYTES):
        raise ValueError("cache must be [num_pages,64,352]")
    B, K = topk.shape
    if page_table.shape[0] != B or seq_lens.shape[0] != B:
        raise ValueError("page_table and seq_lens need one row per sequence")
    pp = (K + PAGE_ROWS - 1) // PAGE_ROWS
    if staged is None:
        staged = torch.empty((B * pp, PAGE_ROWS, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    else:
        _req(staged, "staged", torch.uint8, 3, dev)
        if tuple(staged.shape) != (B * pp, PAGE_ROWS, FP8_ROW_BYTES):
            raise ValueError("staged must be [B*ceil(K/64),64,576]")
    if staged_topk is None:
        staged_topk = torch.empty((B, K), dtype=torch.int32, device=dev)
    else:
        _req(staged_topk, "staged_topk", torch.int32, 2, dev)
        if tuple(staged_topk.shape) != (B, K):
            raise ValueError("staged_topk must be [B,K]")
    _check(lib.smla_stage_rows_fp8(cache.data_ptr(), cache.shape[0], page_table.data_ptr(),
                                   page_table.shape[1], seq_lens.data_ptr(), topk.data_ptr(), B, K,
                                   staged.data_ptr(), staged_topk.data_ptr(),
                                   _stream_ptr(dev, stream)))
    return staged, staged_topk


def sparse_mla_decode_staged(q: torch.Tensor, cache: torch.Tensor, page_table: torch.Tensor,
                             seq_lens: torch.Tensor, topk: torch.Tensor, softmax_scale: float,
                             out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                             staged: torch.Tensor | None = None,
                             staged_topk: torch.Tensor | None = None,
                             workspace: torch.Tensor | None = None, stream=None):
    """The staged path end to end: stage_rows_fp8, then sparse_mla_decode_fp8
    over the copy.  Returns (out, lse)."""
    staged, staged_topk = stage_rows_fp8(cache, page_table, seq_lens, topk, staged, staged_topk,
                                         stream)
    spt, ssl = staged_tables(topk.shape[0], topk.shape[1], cache.device)
    return sparse_mla_decode_fp8(q, staged, spt, ssl, staged_topk, softmax_scale, out=out,
                                 lse=lse, workspace=workspace, stream=stream)


_topk_workspaces: dict = {}


def topk_workspace(device: torch.device, batch: int, ld: int, stream=None) -> torch.Tensor:
    """A zero-filled top-k workspace for `batch` rows of `ld` scores, cached
    per (device, stream); every select leaves it all zero again."""
    need = int(lib.smla_topk_workspace_bytes(batch, ld))
    key = (device.index, _stream_ptr(device, stream))
    with _ws_lock:
        ws = _topk_workspaces.get(key)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=device)
            _topk_workspaces[key] = ws
        return ws


def topk_select(scores: torch.Tensor, seq_lens: torch.Tensor, topk: int,
                out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """scores [B, ld] fp32 (ld a multiple of 4), seq_lens [B] int32 ->
    [B, topk] int32: the positions of the min(topk, L_b) largest scores of
    each row (unordered), then -1."""
    _req(scores, "scores", torch.float32, 2)
    dev = scores.device
    _req(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, ld = scores.shape
    if seq_lens.shape[0] != B:
        raise ValueError("seq_lens needs one entry per row of scores")
    if out is None:
        out = torch.empty((B, topk), dtype=torch.int32, device=dev)
    else:
        _req(out, "out", torch.int32, 2, dev)
        if tuple(out.shape) != (B, topk):
            raise ValueError("out must be [B, topk]")
    if workspace is None:
        workspace = topk_workspace(dev, B, ld, stream)
    ws_ptr, ws_bytes = _req_workspace(workspace, dev)
    _check(lib.smla_topk_select(scores.data_ptr(), ld, seq_lens.data_ptr(), B, int(topk),
                                out.data_ptr(), ws_ptr, ws_bytes, _stream_ptr(dev, stream)))
    return out


def decode_workspace_bytes_mtp(batch: int, tokens: int, heads: int, topk: int) -> int:
    return int(lib.smla_decode_workspace_bytes_mtp(batch, tokens, heads, topk))


def sparse_mla_decode_mtp(q: torch.Tensor, cache: torch.Tensor, page_table: torch.Tensor,
                          seq_lens: torch.Tensor, topk: torch.Tensor, softmax_scale: float,
                          out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                          workspace: torch.Tensor | None = None, stream=None):
    """Multi-token decode: q [B,T,H,576] bf16, topk [B,T,K] int32, the page
    table and seq_lens per sequence (token j sees [0, L_b - (T-1-j))).
    Returns (out [B,T,H,512] fp32, lse [B,T,H] fp32)."""
    _req(cache, "cache", torch.uint8, 3)
    dev = cache.device
    _req(q, "q", torch.bfloat16, 4, dev)
    _req(page_table, "page_table", torch.int32, 2, dev)
    _req(seq_lens, "seq_lens", torch.int32, 1, dev)
    _req(topk, "topk", torch.int32, 3, dev)
    B, T, H, D = q.shape
    if D != DIM:
        raise ValueError("q must be [B,T,H,576]")
    if tuple(cache.shape[1:]) != (PAGE_ROWS, ROW_BYTES):
        raise ValueError("cache must be [num_pages,64,352]")
    if page_table.shape[0] != B or seq_lens.shape[0] != B or tuple(topk.shape[:2]) != (B, T):
        raise ValueError("page_table, seq_lens per sequence; topk [B,T,K]")
    K = topk.shape[2]
    if out is None:
        out = torch.empty((B, T, H, LATENT), dtype=torch.float32, device=dev)
    else:
        _req_shape(out, "out", torch.float32, (B, T, H, LATENT), dev)
    if lse is None:
        lse = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    else:
        _req_shape(lse, "lse", torch.float32, (B, T, H), dev)
    need = decode_workspace_bytes_mtp(B, T, H, K)
    if workspace is None and need > 0:
        workspace = workspace_for(dev, need, stream)
    ws_ptr, ws_bytes = _req_workspace(workspace, dev)
    _check(lib.smla_sparse_mla_decode_mtp(q.data_ptr(), cache.data_ptr(), cache.shape[0],
                                          page_table.data_ptr(), page_table.shape[1],
                                          seq_lens.data_ptr(), topk.data_ptr(), B, T, H, K,
                                          float(softmax_scale), out.data_ptr(), lse.data_ptr(),
                                          ws_ptr, ws_bytes, _stream_ptr(dev, stream)))
    return out, lse
