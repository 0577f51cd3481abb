"""The hot path under HIP graph capture: a decode step (append + decode, and
the same as one fused call) and a select + decode step are captured once and replayed several times, with the
program's own eager work and synchronisations between the replays (the calls
use no memset, allocation or host sync).  Every replay must equal the eager
result: bit for bit for the decode over a fixed list (deterministic), as a
set for the select (its order is unspecified), and up to the rounding a
list's order moves for the decode over the selected list."""
import numpy as np
import pytest
import torch

import workloads as wl
from cases import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def smla():
    import sparse_mla_decode_amd as m
    return m


def test_stream_pointer_follows_current_stream(dev, smla):
    """The binding launches on torch's current stream: the default one, and a
    side stream made current by torch.cuda.stream."""
    assert smla._stream_ptr(dev) == torch.cuda.current_stream(dev).cuda_stream
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        assert smla._stream_ptr(dev) == s.cuda_stream
        assert smla._stream_ptr(dev) == torch.cuda.current_stream(dev).cuda_stream
    assert smla._stream_ptr(dev) == torch.cuda.current_stream(dev).cuda_stream
    assert smla._stream_ptr(dev, s) == s.cuda_stream


def test_graph_replays_equal_eager(dev, smla):
    note("graph capture of append + decode and select + decode")
    w = wl.WORKLOADS["tp4"]
    lens = wl.context_lengths(w, 0)
    pt_np, num_pages = wl.build_page_table(w, lens, 0)
    cache = torch.zeros((num_pages, 64, 352), dtype=torch.uint8, device=dev)
    wl.fill_cache(w, 0, lens, pt_np, lambda r, s: smla.kv_quant_append(r, s, cache), dev, tail=1)
    rows, slots = wl.tail_rows(w, 0, lens, pt_np, dev, 1)
    pt = torch.as_tensor(pt_np, device=dev)
    sl = torch.as_tensor(lens.astype(np.int32), device=dev)
    tk = torch.as_tensor(wl.topk_indices(w, lens, 0), device=dev)
    q = wl.queries(w, 0, device=dev)
    scores = wl.index_scores(w, lens, 0, device=dev)
    B, H = w.batch, w.heads
    out = torch.empty((B, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    out2 = torch.empty_like(out)
    lse2 = torch.empty_like(lse)
    out3 = torch.empty_like(out)
    lse3 = torch.empty_like(lse)
    sel = torch.empty((B, w.topk), dtype=torch.int32, device=dev)
    ws = torch.zeros(max(smla.decode_workspace_bytes(B, H, w.topk), 256), dtype=torch.uint8,
                     device=dev)
    ws2 = torch.zeros_like(ws)
    ws3 = torch.zeros_like(ws)
    tws = smla.topk_workspace(dev, B, scores.shape[1])

    def step(s):
        smla.kv_quant_append(rows, slots, cache, stream=s)
        smla.sparse_mla_decode(q, cache, pt, sl, tk, w.softmax_scale, out=out, lse=lse,
                               workspace=ws, stream=s)
        # the fused call appends the same rows again (the same bytes) and
        # decodes the same lists: out3, lse3 equal out, lse bit for bit
        smla.append_decode(rows, slots, q, cache, pt, sl, tk, w.softmax_scale, out=out3,
                           lse=lse3, workspace=ws3, stream=s)
        smla.topk_select(scores, sl, w.topk, out=sel, workspace=tws, stream=s)
        smla.sparse_mla_decode(q, cache, pt, sl, sel, w.softmax_scale, out=out2, lse=lse2,
                               workspace=ws2, stream=s)

    # eager reference
    step(None)
    torch.cuda.synchronize(dev)
    ref = [t.clone() for t in (out, lse, out2, lse2)]
    assert torch.equal(out3, ref[0]) and torch.equal(lse3, ref[1]), "eager fused call"
    ref_sel = torch.sort(sel, dim=1).values.clone()

    def rel(a, b):
        return float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))

    # capture on a side stream, as torch requires
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step(s)                                       # warm-up on the capture stream
        torch.cuda.synchronize(dev)
        with torch.cuda.graph(g, stream=s):
            step(s)
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize(dev)
    for rep in range(5):
        for t in (out, lse, out2, lse2, out3, lse3, sel):
            t.fill_(-1 if t.dtype == torch.int32 else float("nan"))
        q.mul_(1.0)                                   # eager work between replays
        torch.cuda.synchronize(dev)
        g.replay()
        torch.cuda.synchronize(dev)
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), "replay %d decode" % rep
        assert torch.equal(out3, ref[0]) and torch.equal(lse3, ref[1]), "replay %d fused" % rep
        assert torch.equal(torch.sort(sel, dim=1).values, ref_sel), "replay %d select" % rep
        # another order of the same list regroups rows into tiles: each f16
        # weight moves by <= 2^-11 relative
        assert rel(out2, ref[2]) < 1e-3, "replay %d select + decode" % rep
        assert float((lse2 - ref[3]).abs().max()) < 1e-3, "replay %d select + decode" % rep
    assert not tws.any(), "the select leaves its workspace all zero"
