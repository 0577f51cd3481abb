"""The decode entry point that allocates nothing (smla_sparse_mla_decode_noalloc),
called through the raw C ABI: its results equal those of smla_sparse_mla_decode
with a caller workspace, on two calls in a row (the second smaller), and a
shape whose partials would not fit the static scratch is refused before
anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

from cases import check_parity, gpu_cache, note, oracle_cache, oracle_decode, small_case, to_dev_bf16

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


def _raw_noalloc(smla, dev, case, cache_d, out, lse):
    """One call of the C entry point with plain device pointers; returns its status."""
    q = to_dev_bf16(case["q"], dev)
    pt = torch.as_tensor(case["pt"], device=dev)
    sl = torch.as_tensor(case["lens"].astype(np.int32), device=dev)
    tk = torch.as_tensor(case["topk"], device=dev)
    raw = ctypes.CDLL(smla.LIB_PATH)
    fn = raw.smla_sparse_mla_decode_noalloc
    P, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    fn.argtypes = [P, P, i64, P, i32, P, P, i32, i32, i32, ctypes.c_float, P, P, P]
    fn.restype = ctypes.c_int
    B, H = q.shape[0], q.shape[1]
    code = fn(q.data_ptr(), cache_d.data_ptr(), cache_d.shape[0], pt.data_ptr(), pt.shape[1],
              sl.data_ptr(), tk.data_ptr(), B, H, tk.shape[1], float(case["scale"]),
              out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)
    return code, (q, pt, sl, tk)


@pytest.mark.parametrize("first,second", [
    ((3, 64, [5000, 3000, 900], 2048), (1, 16, [4096], 256)),
    ((40, 16, [1200 + 97 * i for i in range(40)], 1024), (2, 64, [333, 129], 17)),
])
def test_noalloc_matches_the_workspace_entry_point(dev, smla, first, second):
    for trial, (batch, heads, lens, topk) in enumerate((first, second)):
        note("noalloc call %d: B=%d H=%d K=%d" % (trial, batch, heads, topk))
        case = small_case(batch, heads, lens, topk, seed=500 + 10 * trial + batch)
        cache_d = gpu_cache(case, dev, smla)
        out = torch.full((batch, heads, 512), 7.0, device=dev)
        lse = torch.full((batch, heads), 7.0, device=dev)
        code, (q, pt, sl, tk) = _raw_noalloc(smla, dev, case, cache_d, out, lse)
        assert code == 0, smla.lib.smla_strerror(code)
        ws = torch.full((max(smla.decode_workspace_bytes(batch, heads, topk), 256),), 0x5A,
                        dtype=torch.uint8, device=dev)
        o_ws, l_ws = smla.sparse_mla_decode(q, cache_d, pt, sl, tk, case["scale"], workspace=ws)
        torch.cuda.synchronize(dev)
        # the same kernels and split plan: bit-identical, hence also within the
        # parity bars of the workspace entry point's result and of the oracle
        assert torch.equal(out, o_ws) and torch.equal(lse, l_ws)
        check_parity(out.cpu().numpy(), o_ws.cpu().numpy().astype(np.float64), lse.cpu().numpy(),
                     l_ws.cpu().numpy().astype(np.float64), "vs workspace entry point")
        ref_o, ref_l = oracle_decode(case, oracle_cache(case))
        check_parity(out.cpu().numpy(), ref_o, lse.cpu().numpy(), ref_l, "vs oracle")


def test_noalloc_refuses_shapes_beyond_its_scratch(dev, smla):
    limit = smla.NOALLOC_SCRATCH_BYTES
    shape = None
    for batch in range(64, 4097):
        if smla.decode_workspace_bytes(batch, 64, 2048) > limit:
            shape = (batch, 64, 2048)
            break
    if shape is None:
        pytest.skip("the split plan needs at most %d bytes of partials at 64 heads, "
                    "within the scratch" % max(smla.decode_workspace_bytes(b, 64, 2048)
                                                for b in range(1, 4097)))
    batch, heads, topk = shape
    note("noalloc refusal: B=%d H=%d K=%d needs %d bytes" %
         (batch, heads, topk, smla.decode_workspace_bytes(batch, heads, topk)))
    case = small_case(1, heads, [2048], topk, seed=9)
    cache_d = gpu_cache(case, dev, smla)
    q = torch.zeros((batch, heads, 576), dtype=torch.bfloat16, device=dev)
    pt = torch.zeros((batch, case["pt"].shape[1]), dtype=torch.int32, device=dev)
    sl = torch.full((batch,), 2048, dtype=torch.int32, device=dev)
    tk = torch.zeros((batch, topk), dtype=torch.int32, device=dev)
    out = torch.full((batch, heads, 512), 7.0, device=dev)
    lse = torch.full((batch, heads), 7.0, device=dev)
    with pytest.raises(smla.SmlaError) as e:
        smla.sparse_mla_decode_noalloc(q, cache_d, pt, sl, tk, case["scale"], out, lse)
    assert e.value.code == -8
    torch.cuda.synchronize(dev)
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
