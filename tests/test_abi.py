"""CPU checks of the C ABI: the library loads, exports what include/smla.h
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "smla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(smla_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    import sparse_mla_decode_amd as smla
    names = declared_functions()
    assert set(names) == set(smla.EXPORTS), names
    raw = ctypes.CDLL(smla.LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name


def test_strerror_and_version():
    import sparse_mla_decode_amd as smla
    for code in list(smla.ERRORS) + [-99, 5]:
        s = smla.lib.smla_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0
    assert smla.version() >= 100


def test_workspace_sizes():
    import sparse_mla_decode_amd as smla
    assert smla.decode_workspace_bytes(0, 64, 2048) == 0
    assert smla.decode_workspace_bytes(4, 32, 2048) == 0          # heads unsupported
    assert smla.decode_workspace_bytes(4, 64, 4096) == 0          # topk too large
    # one sequence with 64 heads is split over many workgroups: f16 partials
    # of at least 16 heads x 512 columns (+ fp32 max and sum) for each of
    # more than one split
    ws = smla.decode_workspace_bytes(1, 64, 2048)
    assert ws >= 2 * (16 * 512 * 2 + 16 * 2 * 4)
    assert ws % 256 == 0
    assert smla.decode_workspace_bytes(64, 64, 2048) % 256 == 0
    # a single 64-entry list cannot be split
    assert smla.decode_workspace_bytes(1, 16, 64) == 0


def test_workspace_sizes_follow_the_plan():
    """The split plan, restated in tests/cases.py (and used there to choose
    shapes that reach given split counts), against the library: the
    workspace a call needs is that plan's f16 partials and fp32 (m, l),
    each 256-byte rounded, or nothing for one split."""
    import sparse_mla_decode_amd as smla
    from cases import decode_plan

    def expect(batch, heads, topk, fp8=False, tokens=1):
        units, s, hg = decode_plan(batch, heads, topk, fp8, tokens)
        if s == 1:
            return 0
        r = lambda x: (x + 255) // 256 * 256
        return r(units * s * hg * 512 * 2) + r(units * s * hg * 2 * 4)
    checked = 0
    for heads in (16, 64):
        for batch in (1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 31, 32, 40, 48, 63, 64, 65, 100, 128,
                      129, 200, 256, 1000):
            for topk in (1, 63, 64, 65, 128, 129, 500, 1000, 1024, 1025, 2047, 2048):
                assert smla.decode_workspace_bytes(batch, heads, topk) == \
                    expect(batch, heads, topk), (batch, heads, topk)
                assert smla.decode_workspace_bytes_fp8(batch, heads, topk) == \
                    expect(batch, heads, topk, fp8=True), (batch, heads, topk)
                for tokens in (2, 4, 16):
                    if batch * tokens <= 65535:
                        assert smla.decode_workspace_bytes_mtp(batch, tokens, heads, topk) == \
                            expect(batch, heads, topk, tokens=tokens), (batch, tokens, heads, topk)
                checked += 1
    assert checked == 2 * 25 * 12


def test_workspace_sizes_fp8():
    import sparse_mla_decode_amd as smla
    assert smla.decode_workspace_bytes_fp8(0, 64, 2048) == 0
    assert smla.decode_workspace_bytes_fp8(4, 32, 2048) == 0
    assert smla.decode_workspace_bytes_fp8(4, 64, 4096) == 0
    # an FP8 workgroup covers at most 1024 list entries: a 2048-entry list is
    # always split in two or more, so even a full batch needs partials
    ws = smla.decode_workspace_bytes_fp8(128, 16, 2048)
    assert ws >= 128 * 2 * (16 * 512 * 2 + 16 * 2 * 4)
    assert ws % 256 == 0
    assert smla.decode_workspace_bytes_fp8(1, 16, 1024) >= 0
    assert smla.decode_workspace_bytes_fp8(1, 16, 64) == 0


FAKE = 0x10000  # never dereferenced: every call below fails host-side validation


def _decode(fmt="", **kw):
    import sparse_mla_decode_amd as smla
    a = dict(q=FAKE, cache=FAKE, num_pages=10, page_table=FAKE, max_pages=4, seq_lens=FAKE,
             topk_indices=FAKE, batch=2, heads=16, topk=64, scale=0.04, out=FAKE, lse=FAKE,
             ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    fn = getattr(smla.lib, "smla_sparse_mla_decode" + fmt)
    return fn(a["q"], a["cache"], a["num_pages"], a["page_table"], a["max_pages"], a["seq_lens"],
              a["topk_indices"], a["batch"], a["heads"], a["topk"], a["scale"], a["out"],
              a["lse"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("fmt", ["", "_fp8"])
def test_decode_rejects_bad_arguments(fmt):
    def d(**kw):
        return _decode(fmt, **kw)
    assert d(heads=32) == -3
    assert d(heads=8) == -3
    assert d(topk=0) == -2
    assert d(topk=2049) == -2
    assert d(batch=0) == -2
    assert d(max_pages=0) == -2
    assert d(num_pages=0) == -2
    assert d(num_pages=(1 << 25) + 1) == -2
    assert d(q=None) == -1
    assert d(cache=None) == -1
    assert d(lse=None) == -1
    assert d(q=FAKE + 2) == -4
    assert d(out=FAKE + 4) == -4
    assert d(cache=FAKE + 16) == -4
    assert d(topk_indices=FAKE + 1) == -4
    # batch 1 x 64 heads needs split partials: missing or short workspace
    assert d(batch=1, heads=64, topk=2048, ws=None, ws_bytes=0) == -5
    assert d(batch=1, heads=64, topk=2048, ws_bytes=1024) == -5
    assert d(batch=1, heads=64, topk=2048, ws=FAKE + 64) == -4
    # valid arguments on a machine without a gfx950 device: refused, nothing launched
    import torch
    if not torch.cuda.is_available():
        assert d() == -7


def test_append_decode_rejects_bad_arguments():
    """The fused entry point: the decode's checks, plus its new rows and
    slots (present, 16- and 4-byte aligned); nothing is launched."""
    import sparse_mla_decode_amd as smla

    def ad(rows=FAKE, slots=FAKE, **kw):
        a = dict(q=FAKE, cache=FAKE, num_pages=10, page_table=FAKE, max_pages=4, seq_lens=FAKE,
                 topk_indices=FAKE, batch=2, heads=16, topk=64, scale=0.04, out=FAKE, lse=FAKE,
                 ws=FAKE, ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return smla.lib.smla_append_decode(
            rows, slots, a["q"], a["cache"], a["num_pages"], a["page_table"], a["max_pages"],
            a["seq_lens"], a["topk_indices"], a["batch"], a["heads"], a["topk"], a["scale"],
            a["out"], a["lse"], a["ws"], a["ws_bytes"], a["stream"])
    assert ad(rows=None) == -1
    assert ad(slots=None) == -1
    assert ad(rows=FAKE + 8) == -4
    assert ad(slots=FAKE + 2) == -4
    assert ad(heads=32) == -3
    assert ad(topk=0) == -2
    assert ad(q=None) == -1
    assert ad(cache=FAKE + 16) == -4
    assert ad(batch=1, heads=64, topk=2048, ws=None, ws_bytes=0) == -5
    import torch
    if not torch.cuda.is_available():
        assert ad() == -7


def _append(fmt="", **kw):
    import sparse_mla_decode_amd as smla
    a = dict(rows=FAKE, n=5, slots=FAKE, cache=FAKE, num_pages=3, stream=None)
    a.update(kw)
    fn = getattr(smla.lib, "smla_kv_quant_append" + fmt)
    return fn(a["rows"], a["n"], a["slots"], a["cache"], a["num_pages"], a["stream"])


@pytest.mark.parametrize("fmt", ["", "_fp8"])
def test_append_rejects_bad_arguments(fmt):
    def ap(**kw):
        return _append(fmt, **kw)
    assert ap(n=-1) == -2
    assert ap(num_pages=0) == -2
    assert ap(rows=None) == -1
    assert ap(slots=None) == -1
    assert ap(rows=FAKE + 8) == -4
    assert ap(cache=FAKE + 128) == -4
    assert ap(slots=FAKE + 2) == -4
    assert ap(n=0, rows=None) == 0          # nothing to do, nothing touched


def test_stage_rejects_bad_arguments():
    import sparse_mla_decode_amd as smla

    def st(**kw):
        a = dict(cache=FAKE, num_pages=10, page_table=FAKE, max_pages=4, seq_lens=FAKE,
                 topk_indices=FAKE, batch=2, topk=64, staged=FAKE, staged_topk=FAKE, stream=None)
        a.update(kw)
        return smla.lib.smla_stage_rows_fp8(a["cache"], a["num_pages"], a["page_table"],
                                            a["max_pages"], a["seq_lens"], a["topk_indices"],
                                            a["batch"], a["topk"], a["staged"], a["staged_topk"],
                                            a["stream"])
    assert st(batch=0) == -2
    assert st(topk=0) == -2
    assert st(topk=2049) == -2
    assert st(max_pages=0) == -2
    assert st(num_pages=0) == -2
    assert st(staged=None) == -1
    assert st(staged_topk=None) == -1
    assert st(cache=None) == -1
    assert st(staged=FAKE + 16) == -4
    assert st(cache=FAKE + 64) == -4
    assert st(staged_topk=FAKE + 2) == -4
    import torch
    if not torch.cuda.is_available():
        assert st() == -7


def test_topk_select_rejects_bad_arguments():
    import sparse_mla_decode_amd as smla
    assert smla.lib.smla_topk_workspace_bytes(0, 4096) == 0
    assert smla.lib.smla_topk_workspace_bytes(1, 0) == 0
    ws1 = smla.lib.smla_topk_workspace_bytes(1, 4096)
    assert ws1 >= 4 * 2048 + 8 * 4096 and ws1 % 256 == 0
    assert smla.lib.smla_topk_workspace_bytes(10, 4096) == 10 * ws1

    def tk(**kw):
        a = dict(scores=FAKE, ld=4096, seq_lens=FAKE, batch=2, topk=2048, out=FAKE, ws=FAKE,
                 ws_bytes=1 << 30, stream=None)
        a.update(kw)
        return smla.lib.smla_topk_select(a["scores"], a["ld"], a["seq_lens"], a["batch"],
                                         a["topk"], a["out"], a["ws"], a["ws_bytes"], a["stream"])
    assert tk(batch=0) == -2
    assert tk(topk=0) == -2
    assert tk(topk=2049) == -2
    assert tk(ld=0) == -2
    assert tk(ld=4098) == -2                  # not a multiple of 4
    assert tk(scores=None) == -1
    assert tk(out=None) == -1
    assert tk(scores=FAKE + 4) == -4
    assert tk(out=FAKE + 2) == -4
    assert tk(ws=None) == -5
    assert tk(ws_bytes=ws1) == -5             # two queries need twice that
    assert tk(ws=FAKE + 128) == -4
    import torch
    if not torch.cuda.is_available():
        assert tk() == -7


def test_binding_refuses_cpu_tensors():
    import torch
    import sparse_mla_decode_amd as smla
    rows = torch.zeros((2, 576), dtype=torch.bfloat16)
    slots = torch.zeros(2, dtype=torch.int32)
    cache = torch.zeros((1, 64, 352), dtype=torch.uint8)
    with pytest.raises(ValueError):
        smla.kv_quant_append(rows, slots, cache)
    with pytest.raises(ValueError):
        smla.kv_quant_append_fp8(rows, slots, torch.zeros((1, 64, 576), dtype=torch.uint8))
