"""Seeded synthetic inputs for sparse NVFP4-MLA decode.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``: it is the
only code that both the oracle side and the HIP side consume.  It holds none
of the method's arithmetic -- only random numbers, shapes, page tables, index
lists and slot mappings.  Everything is a pure function of (workload, seed,
set id), so any part of an input can be regenerated on its own.

Workload shapes follow the agent-decode shapes the pages describe (a
~140K-token context growing by a ~6K-token tail per turn, top-k 2048 from the
sparse indexer, 64 absorbed heads or a 16-head TP4 share, 64-token pages):
"Prime Inference: serving GLM-5.3 to agents is a KV-cache problem", sections
"The workload", "Decode: TP4, and the copies it keeps" and "Moving the cache:
32K copies for one request".

Recipe (stated once here, repeated in the design notes):
  * KV rows: N(0,1) in fp32 from torch's seeded generator, rounded to BF16
    (round to nearest even); where a workload has outliers, 8 distinct
    channels of the 576, drawn from the seed, are multiplied by 8 (exact).
    Rows are generated in chunks of ``ROW_CHUNK`` tokens per sequence, each
    chunk from its own seed, so any chunk can be regenerated alone.
  * Queries: N(0,1) BF16, shape [B, H, 576].
  * Page tables: ``identity`` (sequence b owns pages in order), ``shuffled``
    (each sequence's own pages in a random order) or ``global`` (one random
    permutation of all physical pages shared out to the sequences).
  * Top-k lists: ``uniform`` = min(K, L) distinct positions uniform over
    [0, L); ``recent`` = K/2 distinct from the last 6000 positions and K/2
    from the rest.  Lists are shuffled (never sorted) and padded with -1 to K.
  * Multi-token (MTP) lists: token 0 takes the workload's list over the
    positions it sees; each draft token j swaps 1 entry in 8 for a fresh
    position among the ones it sees (see ``mtp_topk``).
  * Indexer scores (input of the top-k select): N(0,1) fp32 per position;
    for ``recent`` workloads the last 6000 positions get +RECENT_SHIFT, which
    puts about half of the top 2048 of a 140K context in that window (the
    shape of the ``recent`` lists).  Rows are [B, ld] with ld = max L rounded
    up to a multiple of 4; positions at or past L_b hold 0.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Iterator, Optional, Tuple

import numpy as np
import torch

LATENT = 512
ROPE = 64
DIM = LATENT + ROPE
PAGE_ROWS = 64
ROW_BYTES = 352
ROW_CHUNK = 8192
TAIL = 6000


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    topk: int
    ctx: int = 0                      # fixed context length (0 when ragged)
    ctx_range: Tuple[int, int] = (0, 0)
    pages: str = "global"            # identity | shuffled | global
    index: str = "uniform"           # uniform | recent
    outliers: bool = False
    append_tail: int = 0             # rows per sequence appended inside a step
    desc: str = ""

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(DIM)


WORKLOADS = {
    "tiny": Workload("tiny", batch=1, heads=16, topk=256, ctx=4096, pages="identity",
                     index="uniform", outliers=True,
                     desc="batch 1, 16 heads, 4096-token context, identity pages, "
                          "top-k 256 distinct uniform, 8 outlier channels x8"),
    "tp4": Workload("tp4", batch=32, heads=16, topk=2048, ctx=32768, pages="shuffled",
                    index="uniform",
                    desc="batch 32, 16 heads (TP4 share), 32768-token contexts, shuffled "
                         "per-sequence pages, top-k 2048 distinct uniform"),
    "allheads": Workload("allheads", batch=64, heads=64, topk=2048, ctx=140000,
                         pages="global", index="recent", outliers=True,
                         desc="batch 64, 64 heads, 140000-token contexts, globally permuted "
                              "pages, top-k 2048 (half from the last 6000 tokens), 8 outlier "
                              "channels x8"),
    "ragged": Workload("ragged", batch=128, heads=16, topk=2048, ctx_range=(1024, 146000),
                       pages="global", index="uniform", append_tail=TAIL,
                       desc="128 sessions, contexts U[1024,146000], 16 heads, top-k "
                            "min(2048,L) padded with -1, 6000-token tail appended first"),
    "million": Workload("million", batch=8, heads=64, topk=2048, ctx=1048576,
                        pages="global", index="uniform", append_tail=TAIL,
                        desc="batch 8, 64 heads, 1048576-token contexts, top-k 2048 uniform, "
                             "6000-token tail appended per sequence"),
}


def _seed(*parts: int) -> int:
    """A 63-bit seed derived from integer parts (numpy SeedSequence)."""
    st = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _rng(*parts: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts]))


def _torch_gen(device, *parts: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


# --------------------------------------------------------------------------
# host-side structure
# --------------------------------------------------------------------------

def context_lengths(w: Workload, seed: int = 0) -> np.ndarray:
    if w.ctx:
        return np.full(w.batch, w.ctx, dtype=np.int64)
    lo, hi = w.ctx_range
    return _rng(seed, 1).integers(lo, hi, endpoint=True, size=w.batch).astype(np.int64)


def build_page_table(w: Workload, lens: np.ndarray, seed: int = 0,
                     pages: Optional[str] = None) -> Tuple[np.ndarray, int]:
    """Returns (page_table [B, max_pages] int32 with -1 for unused, num_pages)."""
    kind = pages or w.pages
    npg = [(int(L) + PAGE_ROWS - 1) // PAGE_ROWS for L in lens]
    total = int(sum(npg))
    maxp = max(npg) if npg else 0
    table = np.full((len(lens), max(maxp, 1)), -1, dtype=np.int32)
    if kind == "global":
        perm = _rng(seed, 4).permutation(total).astype(np.int32)
    else:
        perm = np.arange(total, dtype=np.int32)
    off = 0
    for b, n in enumerate(npg):
        ids = perm[off:off + n].copy()
        if kind == "shuffled":
            ids = ids[_rng(seed, 5, b).permutation(n)]
        table[b, :n] = ids
        off += n
    return table, total


def topk_indices(w: Workload, lens: np.ndarray, seed: int = 0, set_id: int = 0,
                 index: Optional[str] = None) -> np.ndarray:
    """[B, K] int32 token positions; unused entries are -1."""
    kind = index or w.index
    K = w.topk
    out = np.full((len(lens), K), -1, dtype=np.int32)
    for b, L in enumerate(lens):
        L = int(L)
        rng = _rng(seed, 2, set_id, b)
        if kind == "recent" and L > TAIL + K // 2:
            half = K // 2
            recent = rng.choice(TAIL, size=half, replace=False) + (L - TAIL)
            older = rng.choice(L - TAIL, size=K - half, replace=False)
            idx = np.concatenate([recent, older])
            idx = idx[rng.permutation(idx.size)]
        else:
            n = min(K, L)
            idx = rng.choice(L, size=n, replace=False)
        out[b, :idx.size] = idx.astype(np.int32)
    return out


MTP_REPLACE = 8     # a draft token's list differs from token 0's in 1 of 8 entries


def mtp_topk(w: Workload, lens: np.ndarray, tokens: int, seed: int = 0,
             set_id: int = 0) -> np.ndarray:
    """[B, T, K] lists of T query tokens per sequence (the accepted token and
    its drafts).  Token 0's list is the workload's list over the positions it
    sees, [0, L - T + 1); token j's list is token 0's with 1 entry in
    MTP_REPLACE swapped for a distinct position drawn from [0, L - T + 1 + j)
    (so drafts share most rows, and may select the newest positions)."""
    B, K = len(lens), w.topk
    base = topk_indices(w, np.maximum(np.asarray(lens) - (tokens - 1), 0), seed, set_id)
    out = np.repeat(base[:, None, :], tokens, axis=1)
    for b in range(B):
        L = int(lens[b])
        for j in range(1, tokens):
            rng = _rng(seed, 6, set_id, b, j)
            row = out[b, j]
            valid = np.flatnonzero(row >= 0)
            vis = max(L - (tokens - 1) + j, 0)
            m = valid.size // MTP_REPLACE
            if m == 0 or vis <= valid.size:
                continue
            taken = set(row[valid].tolist())
            fresh = []
            while len(fresh) < m:
                t = int(rng.integers(0, vis))
                if t not in taken:
                    taken.add(t)
                    fresh.append(t)
            row[rng.choice(valid, size=m, replace=False)] = fresh
    return out.astype(np.int32)


def outlier_channels(w: Workload, seed: int = 0) -> np.ndarray:
    if not w.outliers:
        return np.zeros(0, dtype=np.int64)
    return np.sort(_rng(seed, 6).choice(DIM, size=8, replace=False)).astype(np.int64)


def slots_for(page_table: np.ndarray, b: int, t0: int, n: int) -> np.ndarray:
    """Cache slots (page * 64 + row) of tokens [t0, t0+n) of sequence b."""
    t = np.arange(t0, t0 + n, dtype=np.int64)
    return (page_table[b, t // PAGE_ROWS].astype(np.int64) * PAGE_ROWS
            + t % PAGE_ROWS).astype(np.int32)


# --------------------------------------------------------------------------
# tensors (torch, on any device)
# --------------------------------------------------------------------------

def kv_chunk(w: Workload, seed: int, b: int, c: int, device="cpu") -> torch.Tensor:
    """Rows of tokens [c*ROW_CHUNK, (c+1)*ROW_CHUNK) of sequence b, [ROW_CHUNK, 576] bf16."""
    g = _torch_gen(device, seed, 7, b, c)
    x = torch.randn((ROW_CHUNK, DIM), generator=g, device=device, dtype=torch.float32)
    x = x.to(torch.bfloat16)
    ch = outlier_channels(w, seed)
    if ch.size:
        idx = torch.as_tensor(ch, device=device)
        x[:, idx] = x[:, idx] * 8
    return x


def kv_rows(w: Workload, seed: int, b: int, t0: int, n: int, device="cpu") -> torch.Tensor:
    """Rows of tokens [t0, t0+n) of sequence b, [n, 576] bf16."""
    parts = []
    t = t0
    while t < t0 + n:
        c = t // ROW_CHUNK
        lo = t - c * ROW_CHUNK
        hi = min(ROW_CHUNK, t0 + n - c * ROW_CHUNK)
        parts.append(kv_chunk(w, seed, b, c, device)[lo:hi])
        t += hi - lo
    if not parts:
        return torch.zeros((0, DIM), dtype=torch.bfloat16, device=device)
    return torch.cat(parts, 0)


def rows_at(w: Workload, seed: int, b: int, positions: np.ndarray, device="cpu") -> torch.Tensor:
    """Rows of the given token positions of sequence b (any order), [n, 576] bf16."""
    positions = np.asarray(positions, dtype=np.int64)
    out = torch.zeros((positions.size, DIM), dtype=torch.bfloat16, device=device)
    chunks = positions // ROW_CHUNK
    for c in np.unique(chunks):
        sel = np.nonzero(chunks == c)[0]
        rows = kv_chunk(w, seed, b, int(c), device)
        out[torch.as_tensor(sel, device=device)] = rows[
            torch.as_tensor(positions[sel] - c * ROW_CHUNK, device=device)]
    return out


def queries(w: Workload, seed: int = 0, set_id: int = 0, device="cpu",
            batch: Optional[int] = None) -> torch.Tensor:
    B = w.batch if batch is None else batch
    g = _torch_gen(device, seed, 3, set_id)
    x = torch.randn((B, w.heads, DIM), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


RECENT_SHIFT = 1.5


def index_scores(w: Workload, lens: np.ndarray, seed: int = 0, set_id: int = 0,
                 device="cpu") -> torch.Tensor:
    """Synthetic indexer scores [B, ld] fp32 (see the recipe above)."""
    ld = int(-(-int(max(int(lens.max()), 1)) // 4) * 4)
    out = torch.zeros((w.batch, ld), dtype=torch.float32, device=device)
    for b in range(w.batch):
        L = int(lens[b])
        if L == 0:
            continue
        g = _torch_gen(device, seed, 5, set_id, b)
        out[b, :L] = torch.randn((L,), generator=g, device=device, dtype=torch.float32)
        if w.index == "recent":
            out[b, max(0, L - TAIL):L] += RECENT_SHIFT
    return out


def iter_fill(w: Workload, seed: int, lens: np.ndarray, page_table: np.ndarray,
              device="cpu", tail: int = 0) -> Iterator[Tuple[int, int, torch.Tensor, np.ndarray]]:
    """Yields (b, t0, rows [n,576] bf16, slots [n] int32) covering tokens
    [0, L_b - tail) of every sequence -- the prefix a setup step fills."""
    for b, L in enumerate(lens):
        end = max(int(L) - tail, 0)
        t = 0
        while t < end:
            c = t // ROW_CHUNK
            n = min(ROW_CHUNK, end - t)
            rows = kv_chunk(w, seed, b, c, device)[:n]
            yield b, t, rows, slots_for(page_table, b, t, n)
            t += n


def fill_cache(w: Workload, seed: int, lens: np.ndarray, page_table: np.ndarray,
               append, device, tail: int = 0) -> int:
    """Fill tokens [0, L_b - tail) of every sequence through ``append(rows,
    slots)`` (the caller's quantise-append).  Returns the number of rows."""
    total = 0
    for b, t0, rows, slots in iter_fill(w, seed, lens, page_table, device, tail):
        append(rows, torch.as_tensor(slots, device=device))
        total += rows.shape[0]
    return total


def tail_rows(w: Workload, seed: int, lens: np.ndarray, page_table: np.ndarray, device,
              tail: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rows and slots of the last min(tail, L_b) tokens of every sequence,
    concatenated: the new tokens one append step writes."""
    rows, slots = [], []
    for b, L in enumerate(lens):
        L = int(L)
        t0 = max(L - tail, 0)
        rows.append(kv_rows(w, seed, b, t0, L - t0, device))
        slots.append(slots_for(page_table, b, t0, L - t0))
    return (torch.cat(rows, 0),
            torch.as_tensor(np.concatenate(slots), device=device))


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """BF16 tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
