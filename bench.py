"""Benchmark of the sparse NVFP4-MLA decode hot path on one MI355X.

One step = one pass of the whole path over one batch: quantise-append of the
newest token's row of every sequence, then sparse MLA decode of one query per
sequence over its top-k rows.  Inputs are resident in HBM before timing
starts.  The timed loop rotates through independent (q, top-k) sets so that
the rows a step reads are not the rows the previous steps left in the 256 MB
Infinity Cache.

Prints ONE JSON line (metric, value = effective KV GB/s over the step, ...,
roofline of the decode kernel, cpu_baseline of the oracle on host cores).
`--format fp8` runs the same step over the lean FP8 cache (576-byte rows);
`--path staged` replaces the fused decode by the staged path (gather-unpack
of the NVFP4 rows into a lean FP8 copy in HBM, then the FP8 decode over it).
`--op select` times the top-k select over the workload's synthetic indexer
scores instead, `--op mtp --tokens T` a multi-token step (T new rows
appended per sequence, then T queries per sequence, each with its own list),
and `--op append` the bulk quantise-append of the workload's tail rows (the
ragged and million configurations); each prints its own JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0           # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0    # MI355X dense FP16/BF16 matrix, published
ROW_BYTES = {"nvfp4": 352, "fp8": 576}          # bytes of one cache row
FLOPS_PER_HEAD_ROW = 2 * 576 + 2 * 512         # score + value contraction
CACHE_BYTES_MALL = 256 << 20

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.txt")
CALIB_FLOATS = 64 << 20          # calibration kernel: y = -x over 256 MiB of fp32


def log(msg):
    sys.stderr.write("[bench] %s\n" % msg)
    sys.stderr.flush()


# the sources each kernel family is compiled from (its .hip file and the
# device headers it includes)
KERNEL_SOURCES = {
    "decode": ("sparse_mla_decode.hip", "decode_device.h", "nvfp4_quant.h", "e4m3.h"),
    "append": ("kv_quant_append.hip", "nvfp4_quant.h", "e4m3.h"),
    "select": ("topk_select.hip", "decode_device.h"),
    "staged": ("stage_rows.hip",),
}


def source_hash(kind: str = "decode") -> str:
    """First 16 hex digits of the sha256 over a kernel family's source files."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "sparse_mla_decode_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def kernel_source_hash() -> str:
    """The decode kernels' source hash (the key of the traffic record)."""
    return source_hash("decode")


def source_hashes() -> dict:
    return {k: source_hash(k) for k in KERNEL_SOURCES}


def traffic_key(workload: str, fmt: str) -> str:
    return workload if fmt == "nvfp4" else workload + "-" + fmt


def measured_traffic(workload: str, full: bool = False):
    """HBM bytes per decode call from committed rocprofv3 counter runs, or None
    when the kernel source changed since they were taken.  The file holds one
    line per workload: `<workload> <source hash> <bytes per call> <fetch>
    <write>`; with full=True the (total, fetch, write) triple."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for ln in lines:
        parts = ln.split()
        if len(parts) >= 5 and parts[0] == workload and not ln.startswith("#"):
            if parts[1] != kernel_source_hash():
                return None
            return (int(parts[2]), int(parts[3]), int(parts[4])) if full else int(parts[2])
    return None


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    return rows


def summarize_kernel_stats(d):
    """Text summary of a rocprofv3 --kernel-trace --stats directory: the
    library's kernels (and the total of one decode call)."""
    rows = _csv_rows(d, "kernel_stats.csv")
    import re
    out = ["# source hashes: " + " ".join("%s=%s" % kv for kv in source_hashes().items()),
           "%-60s %8s %12s %12s %12s" % ("kernel", "calls", "avg_us", "min_us", "max_us")]
    for r in rows:
        name = r["Name"]
        if "smla" not in name:
            continue
        # demangled (smla::(anonymous namespace)::k<2, 1>(...)) or mangled
        # (_ZN4smla12_GLOBAL__N_11kILi2ELi1EEEv...) names -> k or k<2, 1>
        m = re.search(r"(kv_quant_append(?:_fp8)?_kernel|sparse_mla_decode_kernel|"
                      r"stage_rows_fp8_kernel|topk_hist_kernel|topk_split_kernel|topk_finish_kernel|"
                      r"merge_splits_kernel)(I(?:L[ib]-?\d+E)+E|<[^>]*>)?", name)
        if not m:
            continue
        targs = m.group(2) or ""
        if targs.startswith("I"):
            targs = "<%s>" % ", ".join(re.findall(r"L[ib](-?\d+)E", targs))
        short = m.group(1) + targs
        out.append("%-60s %8s %12.3f %12.3f %12.3f" % (
            short[:60], r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
            float(r["MaxNs"]) / 1e3))
    return "\n".join(out)


def summarize_counters(fetch_dir, write_dir, workload):
    """HBM bytes per decode call from two rocprofv3 --pmc runs (FETCH_SIZE,
    then WRITE_SIZE, both in KiB per dispatch), each scaled by what the same
    counter reads for the calibration kernel (y = -x over 256 MiB fp32: reads
    256 MiB, writes 256 MiB)."""
    res = {}
    for d, counter in ((fetch_dir, "FETCH_SIZE"), (write_dir, "WRITE_SIZE")):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] != counter:
                continue
            per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        calib = [v for k, vs in per.items() if "neg" in k for v in vs]
        # the plain decode call only: a fused append-and-decode dispatch
        # (template flag true: demangled "true>", mangled "Lb1E") also
        # quantises and stores the step's new rows
        dec = [v for k, vs in per.items() if "sparse_mla_decode_kernel" in k
               and "true>" not in k and "Lb1E" not in k for v in vs]
        mrg = [v for k, vs in per.items() if "merge_splits_kernel" in k for v in vs]
        if not calib or not dec:
            raise SystemExit("missing calibration or decode dispatches in %s" % d)
        kib_true = CALIB_FLOATS * 4 / 1024.0
        factor = kib_true / (sum(calib) / len(calib))
        dec_kib = sum(dec) / len(dec)
        mrg_kib = sum(mrg) / len(mrg) if mrg else 0.0
        res[counter] = (factor, dec_kib, mrg_kib, len(dec))
    fb = (res["FETCH_SIZE"][1] + res["FETCH_SIZE"][2]) * res["FETCH_SIZE"][0] * 1024
    wb = (res["WRITE_SIZE"][1] + res["WRITE_SIZE"][2]) * res["WRITE_SIZE"][0] * 1024
    lines = ["# counter  factor  decode_KiB/dispatch  merge_KiB/dispatch  dispatches"]
    for c, (f, dk, mk, n) in res.items():
        lines.append("# %-10s %.4f %14.1f %14.1f %6d" % (c, f, dk, mk, n))
    lines.append("# workload  source_hash  hbm_bytes_per_call  fetch_bytes  write_bytes")
    fb, wb = int(fb), int(wb)  # the total is the sum of the recorded parts
    lines.append("%s %s %d %d %d" % (workload, kernel_source_hash(), fb + wb, fb, wb))
    return "\n".join(lines)


def step_fusable(args, w) -> bool:
    """A decode step can be one append_decode call: NVFP4 rows, the fused
    decode path, and one new row per sequence (the workloads whose step
    appends no multi-row tail)."""
    return (args.op == "decode" and args.format == "nvfp4" and args.path == "fused"
            and not w.append_tail)


def warm_clocks(fn, seconds):
    """Untimed calls fn(0), fn(1), ... until `seconds` of wall time have
    passed, then a synchronisation: the GPU's clocks rise over the first tens
    of milliseconds of sustained load (a cold first run of 200 allheads steps
    averages ~15% slower than the third), and the timed steps should see the
    clocks a serving loop runs at.  Part of the set-up, before the warm-up
    steps."""
    import torch
    if seconds <= 0:
        return
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def events_ms(fn, n):
    """Mean milliseconds per call of fn(0 .. n-1), from two HIP events on the
    current stream (the stream the library launches on) around the n calls,
    with a synchronisation before and after."""
    import torch
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


COPY_BYTES = 1 << 30             # stream-copy denominator: 1 GiB read + 1 GiB written
FLUSH_BYTES = 1 << 30            # scratch written between launches in the flush cross-check


def stream_copy_gbps(dev, reps: int = 20) -> float:
    """HBM bandwidth of a plain device copy measured on this GPU: 1 GiB copied
    reps times back to back, read + written bytes over the HIP-event time."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    ms = events_ms(lambda i: b.copy_(a), reps)
    del a, b
    return 2 * COPY_BYTES / (ms * 1e-3) / 1e9


def flushed_median_us(fn, n: int, dev) -> float:
    """Median per-launch time (us) of fn(i) when 1 GiB of scratch is read
    before each launch, so that nothing a launch reads or writes is left in
    the L2s or the Infinity Cache by the launches before it.  A read, not a
    write: a written flush leaves dirty lines whose write-back would fall
    inside the timed launch.  Each launch is bracketed by its own pair of
    HIP events."""
    import torch
    scratch = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        scratch.sum()
        e0.record()
        fn(i)
        e1.record()
    torch.cuda.synchronize()
    del scratch
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3


def summarize_pmc(dirs):
    """Per-kernel averages per dispatch of the counters in one or more
    rocprofv3 --pmc directories, and what they imply.  GRBM_GUI_ACTIVE as
    collected is the sum over the 8 XCDs' GRBM instances, so one XCD's busy
    cycles are a eighth of it.  MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES /
    (one XCD's GRBM_GUI_ACTIVE x 1024 SIMDs); LDS bank-conflict share =
    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; per-wave issue shares =
    SQ_ACTIVE_INST_x / SQ_WAVE_CYCLES (both counted per wave)."""
    import re
    per = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            m = re.search(r"(sparse_mla_decode_kernel|merge_splits_kernel|kv_quant_append(?:_fp8)?_kernel|"
                          r"stage_rows_fp8_kernel|topk_hist_kernel|topk_split_kernel|topk_finish_kernel)",
                          r["Kernel_Name"])
            if not m:
                continue
            per.setdefault(m.group(1), {}).setdefault(r["Counter_Name"], []).append(
                float(r["Counter_Value"]))
    out = []
    for k, cs in sorted(per.items()):
        out.append(k)
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        for c in sorted(avg):
            out.append("  %-28s %16.1f  (%d dispatches)" % (c, avg[c], len(cs[c])))
        g = avg.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        if g:
            out.append("  => one XCD busy %.0f cycles" % g)
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            out.append("  => MFMA busy %.1f%% of SIMD cycles" % (100 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024)))
        if avg.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in avg:
            out.append("  => LDS bank conflicts %.1f%% of LDS active cycles"
                       % (100 * avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_LDS_IDX_ACTIVE"]))
        wc = avg.get("SQ_WAVE_CYCLES")
        if wc:
            for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY",
                      "SQ_WAIT_ANY"):
                if c in avg:
                    out.append("  => %s %.1f%% of wave cycles" % (c, 100 * avg[c] / wc))
    return "\n".join(out)


HOST_SHARE = 16                  # host cores that go with one GPU on the measurement hosts


def host_threads():
    """(threads for the oracle, cores in this process's affinity): all
    affinity cores, but at most one GPU's share of the host (16), so that a
    one-GPU run does not oversubscribe the cores that belong to the other
    GPUs of the host."""
    aff = len(os.sched_getaffinity(0))
    return min(aff, HOST_SHARE), aff


def cpu_baseline(w, seed, lens, tk_np, qbits, budget_s, dev, fmt):
    """Time the oracle's decode on host cores over as many sequences as fit in
    roughly budget_s seconds (at least one)."""
    import torch
    import oracle
    import workloads as wl
    cores, aff = host_threads()
    quant = oracle.quant_rows if fmt == "nvfp4" else oracle.quant_rows_fp8
    rb = ROW_BYTES[fmt]
    prepared = {}  # sequence -> (its selected rows as a small cache, row count)

    def prepare(b):
        sel = tk_np[b][tk_np[b] >= 0].astype(np.int64)
        sel = sel[sel < lens[b]]
        n = sel.size
        rows = quant(wl.bf16_bits(wl.rows_at(w, seed, b, sel, device=dev)))
        mini = np.zeros(((max(n, 1) + 63) // 64, 64, rb), dtype=np.uint8)
        mini.reshape(-1, rb)[:n] = rows
        return mini, n

    # the batch's sequences in turn, again from the first once all are done,
    # until the time budget is used (the inputs of each are built once,
    # outside the timing)
    done, t_used, kv_bytes = 0, 0.0, 0
    while t_used < budget_s:
        b = done % w.batch
        if b not in prepared:
            prepared[b] = prepare(b)
        mini, n = prepared[b]
        pt = np.arange(mini.shape[0], dtype=np.int32)[None]
        t0 = time.perf_counter()
        oracle.sparse_mla_decode(qbits[b:b + 1], mini, pt, np.array([n]),
                                 np.arange(n, dtype=np.int32)[None], w.softmax_scale,
                                 nthreads=cores)
        t_used += time.perf_counter() - t0
        done += 1
        kv_bytes += n * rb
    gbps = kv_bytes / t_used / 1e9
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": min(cores, w.heads), "kind": "oracle",
            "sample": "oracle decode (fp64 C, OpenMP over heads, %d threads of %d affinity cores), "
                      "%d query decodes over %d of the %d sequences (%d heads, %d selected rows "
                      "each), %.1f s; %.2f queries/s"
                      % (cores, aff, done, len(prepared), w.batch, w.heads,
                         int(np.mean([min(w.topk, L) for L in lens])), t_used, done / t_used)}


def bench_select(args, w, dev):
    """Time the top-k select over R rotating sets of synthetic indexer scores."""
    import torch
    import sparse_mla_decode_amd as smla
    import workloads as wl
    lens = wl.context_lengths(w, args.seed)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    first = wl.index_scores(w, lens, args.seed, 0, device=dev)
    set_bytes = first.numel() * 4
    sets = args.sets or max(2, math.ceil(2 * CACHE_BYTES_MALL / set_bytes) + 1)
    scores = [first] + [wl.index_scores(w, lens, args.seed, s, device=dev) for s in range(1, sets)]
    out = torch.empty((w.batch, w.topk), dtype=torch.int32, device=dev)
    ws = smla.topk_workspace(dev, w.batch, first.shape[1])
    log("select %s: %d x %d scores, %d rotating sets" % (w.name, w.batch, first.shape[1], sets))
    warm_clocks(lambda i: smla.topk_select(scores[i % sets], sl, w.topk, out=out, workspace=ws),
                args.warm_seconds)
    for i in range(args.warmup):
        smla.topk_select(scores[i % sets], sl, w.topk, out=out, workspace=ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        smla.topk_select(scores[(args.warmup + i) % sets], sl, w.topk, out=out, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    # algorithmic bytes: every valid score read once, the lists written once
    alg = float(np.minimum(lens, first.shape[1]).sum()) * 4 + w.batch * w.topk * 4
    gbps = alg / (us * 1e-6) / 1e9
    result = {
        "metric": "top-k select of indexer scores: scores GB/s and queries/sec",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warm_seconds": args.warm_seconds, "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "topk": w.topk,
                   "scores_per_query": int(first.shape[1]), "rotating_sets": sets},
        "select_us": round(us, 2), "queries_per_s": round(w.batch / (us * 1e-6), 1),
        "source_hashes": source_hashes(),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu:
        from concurrent.futures import ThreadPoolExecutor
        import oracle
        x = first.cpu().numpy()
        cores, aff = host_threads()
        # the oracle's select of one query per call (a qsort on one thread),
        # `cores` calls at a time on a thread pool (a foreign call through
        # ctypes releases the GIL), the batch's queries in turn, until the
        # time budget is used
        done, dt, cbytes = 0, 0.0, 0.0
        with ThreadPoolExecutor(max_workers=cores) as pool:
            while dt < args.cpu_budget:
                idx = [(done + i) % w.batch for i in range(cores)]
                t = time.perf_counter()
                list(pool.map(lambda q: oracle.topk_select(x[q:q + 1], lens[q:q + 1], w.topk), idx))
                dt += time.perf_counter() - t
                done += len(idx)
                cbytes += float(sum(min(int(lens[q]), x.shape[1]) for q in idx)) * 4
        result["cpu_baseline"] = {"value": round(cbytes / dt / 1e9, 4), "unit": "GB/s",
                                  "cores": cores, "kind": "oracle",
                                  "sample": "oracle select (a qsort per query, one query per call) "
                                            "on %d threads of %d affinity cores, %d query selects "
                                            "over the %d queries, %.1f s; %.1f queries/s"
                                            % (cores, aff, done, w.batch, dt, done / dt)}
    print(json.dumps(result), flush=True)


def bench_mtp(args, w, dev):
    """An MTP verification step: append the T newest rows of every sequence,
    then decode T query tokens per sequence, each over its own list."""
    import torch
    import sparse_mla_decode_amd as smla
    import workloads as wl
    T = args.tokens
    lens = wl.context_lengths(w, args.seed)
    pt_np, num_pages = wl.build_page_table(w, lens, args.seed)
    cache = torch.zeros((num_pages, 64, 352), dtype=torch.uint8, device=dev)
    wl.fill_cache(w, args.seed, lens, pt_np, lambda r, s_: smla.kv_quant_append(r, s_, cache), dev)
    rows, slots = wl.tail_rows(w, args.seed, lens, pt_np, dev, T)
    pt = torch.as_tensor(pt_np, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    per_set = int(sum(min(w.topk, int(L)) for L in lens)) * T * 352
    sets = args.sets or max(4, math.ceil(2 * CACHE_BYTES_MALL / per_set) + 1)
    qs, tks, nvalid, nuniq = [], [], [], []
    for st in range(sets):
        tk = wl.mtp_topk(w, lens, T, args.seed, st)
        nvalid.append(int((tk >= 0).sum()))
        nuniq.append(sum(len(np.unique(tk[b][tk[b] >= 0])) for b in range(w.batch)))
        tks.append(torch.as_tensor(tk, device=dev))
        qs.append(torch.cat([wl.queries(w, args.seed, set_id=1000 * st + j, device=dev)[:, None]
                             for j in range(T)], 1).contiguous())
    out = torch.empty((w.batch, T, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, T, w.heads), dtype=torch.float32, device=dev)
    ws = torch.zeros(max(smla.decode_workspace_bytes_mtp(w.batch, T, w.heads, w.topk), 256),
                     dtype=torch.uint8, device=dev)
    log("mtp %s T=%d: %d sets, %d rows appended per step" % (w.name, T, sets, rows.shape[0]))

    def decode_call(i):
        st = i % sets
        smla.sparse_mla_decode_mtp(qs[st], cache, pt, sl, tks[st], w.softmax_scale, out=out,
                                   lse=lse, workspace=ws)

    def step(i):
        smla.kv_quant_append(rows, slots, cache)
        decode_call(i)
    warm_clocks(step, args.warm_seconds)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    events_ms(lambda i: step(args.warmup + i), args.steps)
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    dec_s = events_ms(lambda i: decode_call(args.warmup + i), args.steps) * 1e-3
    used = [(args.warmup + i) % sets for i in range(args.steps)]
    dec_bytes = float(np.mean([nvalid[u] for u in used])) * 352
    uniq_bytes = float(np.mean([nuniq[u] for u in used])) * 352
    flops = float(np.mean([nvalid[u] for u in used])) * w.heads * FLOPS_PER_HEAD_ROW
    app_bytes = rows.shape[0] * (576 * 2 + 352)
    gbps = dec_bytes / dec_s / 1e9
    tflops = flops / dec_s / 1e12
    result = {
        "metric": "multi-token sparse NVFP4-MLA decode: effective KV GB/s and queries/sec",
        "value": round((dec_bytes + app_bytes) / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "warm_seconds": args.warm_seconds, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "tokens": T, "heads": w.heads,
                   "topk": w.topk, "rotating_sets": sets},
        "decode_us": round(dec_s * 1e6, 2), "decode_kv_GBps": round(gbps, 1),
        "unique_rows_frac": round(uniq_bytes / dec_bytes, 4),
        "decode_tflops": round(tflops, 2),
        "queries_per_s": round(w.batch * T / (ms * 1e-3), 1),
        "source_hashes": source_hashes(),
        "roofline": ({"bound": "hbm", "achieved": round(uniq_bytes / dec_s / 1e9, 1),
                      "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                      "frac": round(uniq_bytes / dec_s / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None}
                     if w.heads * FLOPS_PER_HEAD_ROW / 352 < MFMA_F16_PEAK_TFLOPS / HBM_PEAK_GBPS * 1e3
                     else {"bound": "mfma", "achieved": round(tflops, 2),
                           "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None}),
    }
    if not args.no_cpu:
        import oracle
        tk0 = tks[0].cpu().numpy()
        qb = wl.bf16_bits(qs[0])
        cores, aff = host_threads()
        prepared = {}  # sequence -> its rows as a small cache, lists, row count, selected rows

        def prepare(b):
            sel_all = [tk0[b, j][tk0[b, j] >= 0].astype(np.int64) for j in range(T)]
            uniq = np.unique(np.concatenate(sel_all))
            rows_ = oracle.quant_rows(wl.bf16_bits(wl.rows_at(w, args.seed, b, uniq, device=dev)))
            n = uniq.size
            mini = np.zeros(((n + 63) // 64, 64, 352), dtype=np.uint8)
            mini.reshape(-1, 352)[:n] = rows_
            where = {int(t): i for i, t in enumerate(uniq)}
            tk_m = np.full((1, T, w.topk), -1, dtype=np.int32)
            for j in range(T):
                tk_m[0, j, :sel_all[j].size] = [where[int(t)] for t in sel_all[j]]
            return mini, tk_m, n, sum(x.size for x in sel_all)

        # the sequences in turn, again from the first once all are done, until
        # the time budget is used (inputs built once, outside the timing)
        t_used, done, kvb = 0.0, 0, 0
        while t_used < args.cpu_budget:
            b = done % w.batch
            if b not in prepared:
                prepared[b] = prepare(b)
            mini, tk_m, n, n_sel = prepared[b]
            t0 = time.perf_counter()
            # every selected row is visible to its token here: lengths n + T - 1
            oracle.sparse_mla_decode_mtp(qb[b:b + 1], mini,
                                         np.arange(mini.shape[0], dtype=np.int32)[None],
                                         np.array([n + T - 1]), tk_m, w.softmax_scale,
                                         nthreads=cores)
            t_used += time.perf_counter() - t0
            done += 1
            kvb += n_sel * 352
        result["cpu_baseline"] = {
            "value": round(kvb / t_used / 1e9, 4), "unit": "GB/s", "cores": min(cores, w.heads),
            "kind": "oracle",
            "sample": "oracle multi-token decode (fp64 C, OpenMP over heads, %d threads of %d "
                      "affinity cores), %d sequence decodes of %d tokens over %d of the %d "
                      "sequences, %.1f s" % (cores, aff, done, T, len(prepared), w.batch, t_used)}
    print(json.dumps(result), flush=True)


def bench_append(args, w, dev):
    """The bulk quantise-append of the workload's tail: the newest
    min(tail, L) tokens of every sequence (ragged, million) or the newest
    token (other workloads), into their cache slots.  Algorithmic bytes: a
    BF16 row read (1,152 B) and a cache row written per row."""
    import torch
    import sparse_mla_decode_amd as smla
    import workloads as wl
    fmt = args.format
    rb = ROW_BYTES[fmt]
    lens = wl.context_lengths(w, args.seed)
    pt_np, num_pages = wl.build_page_table(w, lens, args.seed)
    cache = torch.zeros((num_pages, 64, rb), dtype=torch.uint8, device=dev)
    tail = w.append_tail if w.append_tail else 1
    rows, slots = wl.tail_rows(w, args.seed, lens, pt_np, dev, tail)
    fn = smla.kv_quant_append if fmt == "nvfp4" else smla.kv_quant_append_fp8
    n = rows.shape[0]
    per_row = 576 * 2 + rb
    log("append %s (%s rows): %d rows, %.1f MB per call" % (w.name, fmt, n, n * per_row / 1e6))
    call = lambda i: fn(rows, slots, cache)
    warm_clocks(call, args.warm_seconds)
    for i in range(args.warmup):
        call(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = events_ms(call, args.steps)
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # the same slots rewritten after a 1 GiB scratch write: no row of the
    # previous call still sits in the Infinity Cache
    flush_us = flushed_median_us(call, min(args.steps, 50), dev)
    copy_gbps = stream_copy_gbps(dev)
    gbps = n * per_row / (ms * 1e-3) / 1e9
    result = {
        "metric": "quantise-append of BF16 KV rows into the paged %s cache: GB/s (%% HBM peak) "
                  "and rows/sec" % ("NVFP4" if fmt == "nvfp4" else "lean FP8"),
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warm_seconds": args.warm_seconds, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "row_format": fmt, "rows": int(n), "bytes_per_row": per_row,
                   "desc": w.desc},
        "append_us": round(ms * 1e3, 2),
        "append_us_flushed_median": round(flush_us, 2),
        "append_GBps_flushed": round(n * per_row / (flush_us * 1e-6) / 1e9, 1),
        "rows_per_s": round(n / (ms * 1e-3), 1),
        "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4),
        "stream_copy_GBps": round(copy_gbps, 1),
        "frac_of_copy": round(gbps / copy_gbps, 4),
        "source_hashes": source_hashes(),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None},
    }
    if not args.no_cpu:
        import oracle
        quant = oracle.quant_rows if fmt == "nvfp4" else oracle.quant_rows_fp8
        bits = wl.bf16_bits(rows)          # host copy, outside the timed region
        cores, aff = host_threads()
        cores = oracle.set_threads(cores)  # the routine's OpenMP loop over rows
        chunk = 4096
        t_used, done = 0.0, 0
        while done < n and t_used < args.cpu_budget:
            part = np.ascontiguousarray(bits[done:done + chunk])
            t = time.perf_counter()
            quant(part)
            t_used += time.perf_counter() - t
            done += part.shape[0]
        result["cpu_baseline"] = {
            "value": round(done * per_row / t_used / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": "oracle quant_rows (C, OpenMP over rows, %d threads of %d affinity cores) "
                      "in 4096-row calls, %d of %d rows, %.1f s; %.0f rows/s"
                      % (cores, aff, done, n, t_used, done / t_used)}
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warm-seconds", type=float, default=0.5,
                    help="untimed steps for this long before the warm-up steps (GPU clock ramp)")
    ap.add_argument("--workload", default="allheads")
    ap.add_argument("--format", choices=("nvfp4", "fp8"), default="nvfp4",
                    help="cache row format: NVFP4 (352 B) or lean FP8 (576 B)")
    ap.add_argument("--op", choices=("decode", "select", "mtp", "append"), default="decode",
                    help="the decode step (default), the top-k select alone, an MTP step, or "
                         "the bulk append of the workload's tail rows")
    ap.add_argument("--tokens", type=int, default=4, help="query tokens per sequence (--op mtp)")
    ap.add_argument("--path", choices=("fused", "staged"), default="fused",
                    help="decode path: the fused kernel, or the staged ablation (NVFP4 only)")
    ap.add_argument("--sets", type=int, default=0, help="rotating (q, top-k) sets (0 = auto)")
    ap.add_argument("--step", choices=("auto", "fused", "two-calls"), default="auto",
                    help="a one-row-per-sequence NVFP4 step as one append_decode call (fused; the "
                         "default where it applies) or as kv_quant_append then the decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run y = -x over 256 MiB first (HBM counter calibration)")
    ap.add_argument("--summarize-kernel-stats", metavar="DIR",
                    help="print a summary of a rocprofv3 --kernel-trace --stats directory")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print per-kernel counter averages of rocprofv3 --pmc directories")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print HBM bytes per decode call from FETCH_SIZE / WRITE_SIZE runs")
    args = ap.parse_args()

    if args.summarize_kernel_stats:
        print(summarize_kernel_stats(args.summarize_kernel_stats))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters,
                                 traffic_key(args.workload, args.format)))
        return

    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import workloads as wl
    w = wl.WORKLOADS[args.workload]
    if args.step == "fused" and not step_fusable(args, w):
        raise SystemExit("--step fused needs the decode op, NVFP4 rows, the fused path and a "
                         "workload that appends one row per sequence per step")

    import torch
    import sparse_mla_decode_amd as smla

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "select":
        bench_select(args, w, dev)
        return
    if args.op == "mtp":
        bench_mtp(args, w, dev)
        return
    if args.op == "append":
        bench_append(args, w, dev)
        return
    fmt = args.format
    if args.path == "staged" and fmt != "nvfp4":
        raise SystemExit("--path staged reads an NVFP4 cache")
    rbytes = ROW_BYTES[fmt]
    append_bytes_per_row = 576 * 2 + rbytes      # BF16 row read + cache row written
    seed = args.seed
    lens = wl.context_lengths(w, seed)
    pt_np, num_pages = wl.build_page_table(w, lens, seed)
    log("workload %s (%s rows): %s; cache %d pages (%.2f GB)" % (
        w.name, fmt, w.desc, num_pages, num_pages * 64 * rbytes / 1e9))
    if args.calibrate_copy:
        a = torch.ones(CALIB_FLOATS, dtype=torch.float32, device=dev)
        b_ = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b_)
        torch.cuda.synchronize()
        del a, b_

    cache = torch.zeros((num_pages, 64, rbytes), dtype=torch.uint8, device=dev)
    append_fn = smla.kv_quant_append if fmt == "nvfp4" else smla.kv_quant_append_fp8
    decode_fn = smla.sparse_mla_decode if fmt == "nvfp4" else smla.sparse_mla_decode_fp8
    ws_fn = smla.decode_workspace_bytes if fmt == "nvfp4" else smla.decode_workspace_bytes_fp8
    append = lambda rows, slots: append_fn(rows, slots, cache)
    t0 = time.time()
    wl.fill_cache(w, seed, lens, pt_np, append, dev, tail=w.append_tail)
    # the step's append: the newest min(tail, L) tokens (ragged, million) or
    # the newest token of every sequence (decode steps of the other workloads)
    step_tail = w.append_tail if w.append_tail else 1
    step_rows, step_slots = wl.tail_rows(w, seed, lens, pt_np, dev, step_tail)
    append(step_rows, step_slots)
    torch.cuda.synchronize()
    log("cache filled in %.1f s; step appends %d rows" % (time.time() - t0, step_rows.shape[0]))

    pt = torch.as_tensor(pt_np, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    per_call_bytes = int(sum(min(w.topk, int(L)) for L in lens)) * rbytes
    sets = args.sets or max(4, math.ceil(2 * CACHE_BYTES_MALL / max(per_call_bytes, 1)) + 1)
    qs, tks, nvalid = [], [], []
    for s in range(sets):
        tk_np = wl.topk_indices(w, lens, seed, set_id=s)
        nvalid.append(int((tk_np >= 0).sum()))
        tks.append(torch.as_tensor(tk_np, device=dev))
        qs.append(wl.queries(w, seed, set_id=s, device=dev))
    out = torch.empty((w.batch, w.heads, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.heads), dtype=torch.float32, device=dev)
    ws_bytes = ws_fn(w.batch, w.heads, w.topk)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    log("%d rotating sets, %.1f MB of selected rows each" % (sets, per_call_bytes / 1e6))
    if args.path == "staged":
        pp = (w.topk + 63) // 64
        staged = torch.empty((w.batch * pp, 64, 576), dtype=torch.uint8, device=dev)
        staged_topk = torch.empty((w.batch, w.topk), dtype=torch.int32, device=dev)
        spt, ssl = smla.staged_tables(w.batch, w.topk, dev)
        ws_bytes = smla.decode_workspace_bytes_fp8(w.batch, w.heads, w.topk)
        ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

        def decode_fn(q_, cache_, pt_, sl_, tk_, scale_, out, lse, workspace):
            smla.stage_rows_fp8(cache_, pt_, sl_, tk_, staged=staged, staged_topk=staged_topk)
            smla.sparse_mla_decode_fp8(q_, staged, spt, ssl, staged_topk, scale_, out=out,
                                       lse=lse, workspace=workspace)

    def decode_call(i):
        s = i % sets
        decode_fn(qs[s], cache, pt, sl, tks[s], w.softmax_scale, out=out, lse=lse, workspace=ws)

    def step_two_calls(i):
        append_fn(step_rows, step_slots, cache)
        decode_call(i)

    # a step that appends one row per sequence (the newest token of each) can
    # be one fused call: the same cache bytes, out and lse as the two calls
    fusable = step_fusable(args, w)
    assert not fusable or step_rows.shape[0] == w.batch
    step_kind = "fused" if (fusable and args.step != "two-calls") else "two-calls"

    def step_fused(i):
        s = i % sets
        smla.append_decode(step_rows, step_slots, qs[s], cache, pt, sl, tks[s], w.softmax_scale,
                           out=out, lse=lse, workspace=ws)

    step = step_fused if step_kind == "fused" else step_two_calls

    warm_clocks(step, args.warm_seconds)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # the timed steps: wall clock between two synchronisations, and two HIP
    # events on the library's stream around them (nothing is recorded between
    # the steps: an event record inside the loop costs the step ~8 us)
    t_start = time.perf_counter()
    gpu_step_ms = events_ms(lambda i: step(args.warmup + i), args.steps)
    t_total = time.perf_counter() - t_start
    ms_per_step = t_total * 1e3 / args.steps
    # the decode call and the append alone, each timed the same way over as
    # many back-to-back calls with the same inputs
    dec_ms = np.array([events_ms(lambda i: decode_call(args.warmup + i), args.steps)])
    app_ms = np.array([events_ms(lambda i: append_fn(step_rows, step_slots, cache), args.steps)])
    # the other route's step time, for comparison
    other_ms = None
    if fusable:
        other = step_two_calls if step_kind == "fused" else step_fused
        other_ms = events_ms(lambda i: other(args.warmup + i), args.steps)

    # algorithmic work per step (mean over the sets the timed steps used)
    used = [(args.warmup + i) % sets for i in range(args.steps)]
    dec_bytes = float(np.mean([nvalid[s] for s in used])) * rbytes
    app_bytes = step_rows.shape[0] * append_bytes_per_row
    dec_flops = float(np.mean([nvalid[s] for s in used])) * w.heads * FLOPS_PER_HEAD_ROW
    value = (dec_bytes + app_bytes) / (ms_per_step * 1e-3) / 1e9
    dec_s = float(dec_ms.mean()) * 1e-3
    dec_gbps = dec_bytes / dec_s / 1e9
    dec_tflops = dec_flops / dec_s / 1e12
    ai = w.heads * FLOPS_PER_HEAD_ROW / rbytes
    ridge = MFMA_F16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    tkey = traffic_key(w.name, fmt) + ("-staged" if args.path == "staged" else "")
    traffic = measured_traffic(tkey)
    traffic_full = measured_traffic(tkey, full=True)
    # a plain copy's bandwidth on this GPU (the second denominator), and the
    # flush cross-check of the call time
    copy_gbps = stream_copy_gbps(dev)
    flush_us = flushed_median_us(decode_call, min(args.steps, 100), dev)
    # all bytes a decode call moves at least once: the selected rows, q, the
    # lists, one page-table entry per valid entry, seq_lens, out and lse, and
    # the split partials written then read back by the merge
    nv_mean = float(np.mean([nvalid[s] for s in used]))
    all_bytes = (dec_bytes + w.batch * w.heads * 576 * 2 + w.batch * w.topk * 4 + nv_mean * 4
                 + w.batch * 4 + w.batch * w.heads * (512 + 1) * 4 + 2 * ws_bytes)
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": round(dec_tflops, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dec_tflops / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}

    result = {
        "metric": ("sparse NVFP4-MLA decode: effective KV GB/s (% HBM peak) and queries/sec"
                   if fmt == "nvfp4" else
                   "sparse MLA decode over lean FP8 rows: effective KV GB/s and queries/sec"),
        "path": args.path,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "warm_seconds": args.warm_seconds,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": w.name, "row_format": fmt, "batch": w.batch, "heads": w.heads, "topk": w.topk,
                   "context": int(lens.max()) if w.ctx == 0 else w.ctx,
                   "append_rows_per_step": int(step_rows.shape[0]),
                   "rotating_sets": sets, "desc": w.desc},
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "queries_per_s": round(w.batch / (ms_per_step * 1e-3), 1),
        "decode_us": round(dec_s * 1e6, 2),
        "decode_kv_GBps": round(dec_gbps, 1),
        "decode_tflops": round(dec_tflops, 2),
        "append_us": round(float(app_ms.mean()) * 1e3, 2),
        "gpu_us_per_step": round(gpu_step_ms * 1e3, 2),
        "step": step_kind,
        ("gpu_us_per_step_two_calls" if step_kind == "fused" else "gpu_us_per_step_fused"):
            (round(other_ms * 1e3, 2) if other_ms is not None else None),
        "decode_us_flushed_median": round(flush_us, 2),
        "stream_copy_GBps": round(copy_gbps, 1),
        "decode_kv_frac_of_copy": round(dec_gbps / copy_gbps, 4),
        "decode_all_bytes": int(all_bytes),
        "decode_all_GBps": round(all_bytes / dec_s / 1e9, 1),
        "overfetch": (round(traffic_full[1] / dec_bytes, 3) if traffic_full else None),
        "source_hashes": source_hashes(),
        "roofline": roof,
    }
    if not args.no_cpu:
        tk0 = wl.topk_indices(w, lens, seed, set_id=0)
        qbits = wl.bf16_bits(qs[0])
        log("timing the oracle on host cores (budget %.0f s)" % args.cpu_budget)
        result["cpu_baseline"] = cpu_baseline(w, seed, lens, tk0, qbits, args.cpu_budget, dev,
                                              fmt)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
