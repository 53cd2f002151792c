"""nvfp4_gemm_ws_noalloc, the allocation-free GEMM entry point (split partial tiles in the
library's own per-device scratch array), called through the C ABI: bit-identical to nvfp4_gemm_ws
with a caller workspace on two calls in a row, the second with a smaller input (which leaves the
first call's partials in the scratch), and within the oracle's bar (tests/gemm_check.py)."""
import ctypes as C

import numpy as np
import pytest
import torch

import workloads as W
from gemm_check import assert_gemm_close

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _oq(q):
    torch.cuda.synchronize()
    return dict(codes=q.codes.cpu().numpy(), scales=q.scales.cpu().numpy(), layout=q.layout,
                s_dec=float(q.s_dec.item()))


def _call(nv, fn, qa, qb, c, *extra):
    da, db = qa.desc(), qb.desc()
    rc = fn(C.byref(da), C.byref(db), c.data_ptr(), nv.F32 if c.dtype == torch.float32 else nv.BF16,
            c.stride(0), *extra, torch.cuda.current_stream().cuda_stream)
    assert rc == nv.OK, nv.lib().nvfp4_status_string(rc)


# first call: 16 tiles split 8 ways (32 MiB of partials); second, smaller: 9 tiles split 4 ways
# (9 MiB), ragged edges, bf16 output; third: no split at all
CALLS = [(1024, 1024, 8192, torch.float32), (600, 700, 4096, torch.bfloat16),
         (256, 512, 1024, torch.float32)]


def test_noalloc_gemm_matches_workspace_gemm(nv, orc):
    L = nv.lib()
    for i, (M, N, K, dt) in enumerate(CALLS):
        qa = nv.quantize_1d(W.act((M, K), 70 + i).to(DEV))
        qb = nv.quantize_1d(W.act((N, K), 80 + i).to(DEV))
        need = nv.gemm_workspace_size(M, N, K)
        assert (need > 0) == (i < 2)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        ref_c = torch.full((M, N), float("nan"), dtype=dt, device=DEV)
        _call(nv, L.nvfp4_gemm_ws, qa, qb, ref_c, ws.data_ptr(), need)
        got = torch.full((M, N), float("nan"), dtype=dt, device=DEV)
        _call(nv, L.nvfp4_gemm_ws_noalloc, qa, qb, got)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           ref_c.view(torch.int16 if dt == torch.bfloat16 else torch.int32)), (M, N, K)
        if dt == torch.float32:
            ref = orc.gemm_f64(_oq(qa), _oq(qb), M, N, K)
            assert_gemm_close(got.cpu().numpy(), ref, f"noalloc {M}x{N}x{K}")


def test_noalloc_gemm_validates_like_gemm(nv):
    """Argument errors return before anything is enqueued, as for nvfp4_gemm."""
    L = nv.lib()
    q = nv.QTensor.empty(64, 64)
    c = torch.empty((64, 64), dtype=torch.float32, device=DEV)
    da = q.desc()
    st = torch.cuda.current_stream().cuda_stream
    assert L.nvfp4_gemm_ws_noalloc(None, C.byref(da), c.data_ptr(), nv.F32, 64, st) == nv.ERR_NULL
    qk = nv.QTensor.empty(64, 32)
    dk = qk.desc()
    assert L.nvfp4_gemm_ws_noalloc(C.byref(da), C.byref(dk), c.data_ptr(), nv.F32, 64, st) == nv.ERR_SHAPE
    assert L.nvfp4_gemm_ws_noalloc(C.byref(da), C.byref(da), c.data_ptr(), 9, 64, st) == nv.ERR_DTYPE
