"""GPU parity of nvfp4_gemm_ws, the GEMM whose partly empty last round of output tiles is split
along K into fp32 partial tiles and added in a fixed order: against the float64 oracle
(tests/gemm_check.py bar), deterministic from call to call, bf16 output equal to the RNE of its
own fp32 output, and identical to nvfp4_gemm when the workspace is missing or too small."""
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


def _ran_split(ws):
    """The workspace, filled with 0xFF bytes (NaN floats) before the call, was written: the last
    round was split and its partial tiles stored there."""
    torch.cuda.synchronize()
    return bool((ws != 0xFF).any())


def _split_rows(c_split, c_whole):
    """Rows where the split result differs from nvfp4_gemm's in some element: rows of split tiles
    (another fp32 addition order changes the last bits of almost every sum)."""
    return torch.nonzero((c_split != c_whole).any(dim=1)).flatten().cpu().numpy()


# (M, N, K, B 16x16): 16 tiles split 8 ways; 12 ragged tiles (M, N not multiples of 256) split 8
# ways; 9 tiles with K = 4096 split 4 ways (16 steps each); a 2D-scaled B operand.
SHAPES = [(1024, 1024, 8192, False), (1000, 520, 8192, False), (600, 700, 4096, False),
          (512, 768, 6144, True)]


@pytest.mark.parametrize("M,N,K,b2d", SHAPES)
def test_split_gemm_matches_oracle(nv, orc, M, N, K, b2d):
    need = nv.gemm_workspace_size(M, N, K)
    assert need > 0, "shape chosen to exercise the split"
    a = W.act((M, K), M + 3)
    qa = nv.quantize_1d(a.to(DEV))
    if b2d:
        qb, _ = nv.quantize_2d(W.weight((N, K), N + 5).to(DEV), transposed=False)
    else:
        qb = nv.quantize_1d(W.act((N, K), N + 5).to(DEV))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    c = nv.gemm(qa, qb, torch.float32, workspace=ws)
    assert _ran_split(ws), "no tile was split"
    ref = orc.gemm_f64(_oq(qa), _oq(qb), M, N, K)
    assert_gemm_close(c.cpu().numpy(), ref, f"split {M}x{N}x{K}")
    # deterministic: the partials are added in a fixed order
    c2 = nv.gemm(qa, qb, torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c, c2)
    # bf16 output is the round-to-nearest-even of the same fp32 sums
    cb = nv.gemm(qa, qb, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))


def test_split_gemm_without_workspace_is_plain_gemm(nv):
    """nvfp4_gemm_ws with no workspace, or one byte too small, is nvfp4_gemm bit for bit."""
    import ctypes as C
    M, N, K = 1024, 1024, 8192
    need = nv.gemm_workspace_size(M, N, K)
    qa = nv.quantize_1d(W.act((M, K), 61).to(DEV))
    qb = nv.quantize_1d(W.act((N, K), 62).to(DEV))
    whole = nv.gemm(qa, qb, torch.float32, split=False)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    da, db = qa.desc(), qb.desc()
    st = torch.cuda.current_stream().cuda_stream
    for ptr, nbytes in ((None, 0), (ws.data_ptr(), need - 1)):
        out = torch.full_like(whole, float("nan"))
        rc = nv.lib().nvfp4_gemm_ws(C.byref(da), C.byref(db), out.data_ptr(), nv.F32,
                                    out.stride(0), ptr, nbytes, st)
        assert rc == nv.OK
        torch.cuda.synchronize()
        assert torch.equal(out, whole)


def test_no_split_shapes_need_no_workspace(nv):
    """Full rounds (tiles a multiple of the compute units), short K, or K % 64 != 0: no split."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert nv.gemm_workspace_size(256 * 16, 256 * (cus // 16), 8192) == 0   # whole rounds
    assert nv.gemm_workspace_size(1024, 1024, 512) == 0                     # 8 steps: too short
    assert nv.gemm_workspace_size(1024, 1024, 8192 + 16) == 0               # K % 64 != 0
    assert nv.gemm_workspace_size(0, 1024, 8192) == 0
    assert nv.gemm_workspace_size(1024, 1024, 8192) == 16 * 8 * 256 * 256 * 4


def test_split_gemm_wgrad_shape(nv, orc):
    """The FFN pair's up-projection wgrad, dW1 [20480 x 5120] with K = 16384 tokens: 1600 output
    tiles leave a last round of 64 on 256 compute units, split 4 ways.  Oracle on 48 rows drawn
    from the split tiles and 16 from the others."""
    T, D, FF = W.CFG5["tokens"], W.CFG5["d_model"], W.CFG5["d_ff"]
    sign, _, sw = W.CFG5["layer_seeds"]["up"]
    dy = W.grad((T, FF), W.CFG5["seeds"][5])
    x = W.act((T, D), W.CFG5["seeds"][0])
    qdyt = nv.hadamard_quantize(dy.to(DEV), sign, nv.SR, sw)
    qxt = nv.hadamard_quantize(x.to(DEV), sign, nv.RNE)
    del dy, x
    need = nv.gemm_workspace_size(FF, D, T)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    c = nv.gemm(qdyt, qxt, torch.float32, workspace=ws)
    assert _ran_split(ws)
    whole = nv.gemm(qdyt, qxt, torch.float32, split=False)
    torch.cuda.synchronize()
    split_rows = _split_rows(c, whole)
    assert len(split_rows) >= 256, len(split_rows)          # the split tiles' sums differ in ulps
    rng = np.random.default_rng(3)
    other = np.setdiff1d(np.arange(FF), split_rows)
    rows = np.sort(np.concatenate([rng.choice(split_rows, 48, replace=False),
                                   rng.choice(other, 16, replace=False)]))
    ref = orc.gemm_f64(_oq(qdyt), _oq(qxt), FF, D, T, rows=rows)
    got = c[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    assert_gemm_close(got, ref, "wgrad 20480x5120x16384 split")


def test_mx_split_gemm_matches_oracle(nv, orc):
    """mxfp4_gemm_ws: 12 tiles of a K % 256 == 0 GEMM split 8 ways (ragged edges), against the
    float64 MXFP4 oracle; deterministic; bf16 = RNE of fp32; too small a workspace = mxfp4_gemm."""
    import ctypes as C
    M, N, K = 1000, 520, 8192
    need = nv.mx_gemm_workspace_size(M, N, K)
    assert need > 0
    qa = nv.mx_quantize_1d(W.act((M, K), 91).to(DEV))
    qb = nv.mx_quantize_1d(W.act((N, K), 92).to(DEV))
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    c = nv.mx_gemm(qa, qb, torch.float32, workspace=ws)
    assert _ran_split(ws)
    oa = dict(codes=qa.codes.cpu().numpy(), scales=qa.scales.cpu().numpy())
    ob = dict(codes=qb.codes.cpu().numpy(), scales=qb.scales.cpu().numpy())
    ref = orc.mx_gemm_f64(oa, ob, M, N, K)
    assert_gemm_close(c.cpu().numpy(), ref, "mx split 1000x520x8192")
    c2 = nv.mx_gemm(qa, qb, torch.float32, workspace=ws)
    cb = nv.mx_gemm(qa, qb, torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(c, c2)
    assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))
    whole = nv.mx_gemm(qa, qb, torch.float32, split=False)
    out = torch.full_like(whole, float("nan"))
    da, db = qa.desc(), qb.desc()
    rc = nv.lib().mxfp4_gemm_ws(C.byref(da), C.byref(db), out.data_ptr(), nv.F32, out.stride(0),
                                ws.data_ptr(), need - 1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == nv.OK and torch.equal(out, whole)
    assert nv.mx_gemm_workspace_size(M, N, K + 128) == 0          # K % 256 != 0: no split
