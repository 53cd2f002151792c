"""GPU parity of the NVFP4 and MXFP4 GEMMs against the float64 oracle on the same (GPU-produced,
bit-identical to the oracle's) quantized operands: relative L2 <= 1e-5 and every element within
1e-5 of its row's largest |value| for fp32 output (tests/gemm_check.py); bf16 output must be the
round-to-nearest-even of the same kernel's fp32 output."""
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
    """Host copy of a GPU QTensor in the oracle's dict form."""
    torch.cuda.synchronize()
    d = dict(codes=q.codes.cpu().numpy(), scales=q.scales.cpu().numpy(), layout=q.layout)
    if q.s_dec is not None:
        d["s_dec"] = float(q.s_dec.item())
    return d


def _check_gemm(nv, orc, qa, qb, rows=None, mx=False, bf16_too=True):
    M, N, K = qa.rows, qb.rows, qa.cols
    gemm = nv.mx_gemm if mx else nv.gemm
    c = gemm(qa, qb, torch.float32)
    oa, ob = _oq(qa), _oq(qb)
    if rows is None:
        ref = (orc.mx_gemm_f64 if mx else orc.gemm_f64)(oa, ob, M, N, K)
        got = c.cpu().numpy().astype(np.float64)
    else:
        ref = (orc.mx_gemm_f64 if mx else orc.gemm_f64)(oa, ob, M, N, K, rows=rows)
        got = c.cpu().numpy().astype(np.float64)[rows]
    err = assert_gemm_close(got, ref, f"M={M} N={N} K={K}")
    if bf16_too:
        cb = gemm(qa, qb, torch.bfloat16)
        torch.cuda.synchronize()
        exp = c.cpu().to(torch.bfloat16)
        assert torch.equal(cb.cpu().view(torch.int16), exp.view(torch.int16))
        # and against the oracle itself: the float64 result rounded to bf16, equal except where
        # the fp32 accumulation lands on the other side of a bf16 rounding point (then one ulp)
        gb = cb.cpu() if rows is None else cb.cpu()[torch.as_tensor(rows)]
        rb = torch.from_numpy(np.ascontiguousarray(ref)).to(torch.float32).to(torch.bfloat16)
        gi = gb.view(torch.int16).to(torch.int32)
        ri = rb.view(torch.int16).to(torch.int32)
        equal = gb.float() == rb.float()                  # +0 and -0 count as equal
        same_sign = (gb.float() * rb.float() > 0) | equal
        assert bool(same_sign.all()), "bf16 output: a sign differs from the oracle's"
        ulps = torch.where(equal, torch.zeros_like(gi), (gi - ri).abs())
        assert int(ulps.max()) <= 1, f"bf16 output: {int(ulps.max())} ulps from the oracle's"
        assert float((ulps == 0).float().mean()) >= 0.999, "bf16 output: too many one-ulp differences"
    return err


def test_gemm_small_square(nv, orc):
    """256x256 fp32 N(0,1) with 1% x50 outliers, both operands 1D RNE; full output."""
    a = W.small_fp32((256, 256), 101)
    b = W.small_fp32((256, 256), 102)
    qa, qb = nv.quantize_1d(a.to(DEV)), nv.quantize_1d(b.to(DEV))
    _check_gemm(nv, orc, qa, qb)


@pytest.mark.parametrize("M,N,K,b2d", [(1, 1, 16, False), (200, 144, 80, True), (33, 300, 48, False),
                                       (257, 255, 4112, False), (64, 512, 1040, True)])
def test_gemm_ragged(nv, orc, M, N, K, b2d):
    a = W.act((M, K), M + K)
    if b2d:
        b = W.weight((N, K), N)
        qb, _ = nv.quantize_2d(b.to(DEV), transposed=False)
    else:
        b = W.act((N, K), N * 7)
        qb = nv.quantize_1d(b.to(DEV))
    qa = nv.quantize_1d(a.to(DEV))
    _check_gemm(nv, orc, qa, qb)


def test_gemm_zero_operand(nv, orc):
    a = torch.zeros((64, 64), dtype=torch.bfloat16, device=DEV)
    b = W.act((32, 64), 3).to(DEV)
    c = nv.gemm(nv.quantize_1d(a), nv.quantize_1d(b))
    torch.cuda.synchronize()
    assert torch.count_nonzero(c).item() == 0


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("off", [8, 3])
def test_gemm_strided_output(nv, mx, dtype, off):
    """C written into a column window of a wider matrix (row stride N + 40, first column at an
    aligned (8) or unaligned (3) element offset): the window equals the contiguous result and
    nothing outside it is touched."""
    M, N, K = 300, 264, 256
    a, b = W.act((M, K), 61).to(DEV), W.act((N, K), 62).to(DEV)
    if mx:
        qa, qb, gemm = nv.mx_quantize_1d(a), nv.mx_quantize_1d(b), nv.mx_gemm
    else:
        qa, qb, gemm = nv.quantize_1d(a), nv.quantize_1d(b), nv.gemm
    ref = gemm(qa, qb, dtype)
    big = torch.full((M, N + 40), -7.0, dtype=dtype, device=DEV)
    gemm(qa, qb, dtype, out=big[:, off:off + N])
    torch.cuda.synchronize()
    assert torch.equal(big[:, off:off + N].cpu(), ref.cpu())
    assert bool((big[:, :off] == -7.0).all()) and bool((big[:, off + N:] == -7.0).all())


def _rows(M, n=256, seed=0):
    return np.sort(np.random.default_rng(seed).choice(M, n, replace=False))


def test_gemm_fprop_full(nv, orc):
    """Y = X W^T: X 8192x4096 (1D RNE), W 4096x4096 (16x16 scales); 256 sampled rows."""
    x = W.act(W.CFG2["x"], W.CFG2["seeds"][0]).to(DEV)
    w = W.weight(W.CFG2["w"], W.CFG2["seeds"][1]).to(DEV)
    qx = nv.quantize_1d(x)
    qw, _ = nv.quantize_2d(w, transposed=False)
    _check_gemm(nv, orc, qx, qw, rows=_rows(8192))


def test_gemm_dgrad_full(nv, orc):
    """dX = dY W: dY 8192x4096 SR, B = the transposed 2D copy of W; 256 sampled rows."""
    dy = W.grad(W.CFG3["dy"], W.CFG3["seed"]).to(DEV)
    w = W.weight(W.CFG2["w"], W.CFG2["seeds"][1]).to(DEV)
    qdy = nv.quantize_1d(dy, rounding=1, seed=W.CFG3["sr_seed"])
    _, qwt = nv.quantize_2d(w, transposed=True)
    _check_gemm(nv, orc, qdy, qwt, rows=_rows(8192, seed=1))


def test_gemm_wgrad_full(nv, orc):
    """dW = dY^T X with the random Hadamard on both operands along 16384 tokens; 128 rows."""
    c = W.CFG4
    x = W.act(c["x"], c["seeds"][0]).to(DEV)
    dy = W.grad(c["dy"], c["seeds"][1]).to(DEV)
    qx = nv.hadamard_quantize(x, c["sign_seed"], rounding=0)
    qdy = nv.hadamard_quantize(dy, c["sign_seed"], rounding=1, seed=c["sr_seed"])
    del x, dy
    _check_gemm(nv, orc, qdy, qx, rows=_rows(4096, 128, seed=2), bf16_too=False)


@pytest.mark.parametrize("M,N,K", [(32, 32, 64), (256, 256, 256), (100, 70, 96), (300, 520, 1056),
                                   (300, 520, 1024), (512, 768, 2048), (40, 600, 128),
                                   (1000, 300, 384), (257, 513, 640), (1, 1, 128), (1, 700, 256),
                                   (530, 1, 384), (777, 1000, 768)])
def test_mx_gemm(nv, orc, M, N, K):
    """K % 256 == 0 takes the two-stage direct-to-LDS kernel (one, three, four and eight K steps),
    other K % 128 == 0 the three-stage one (one, three and five steps), both with ragged M and N;
    other K the guarded kernel."""
    a = W.act((M, K), 51)
    b = W.act((N, K), 52)
    qa, qb = nv.mx_quantize_1d(a.to(DEV)), nv.mx_quantize_1d(b.to(DEV))
    _check_gemm(nv, orc, qa, qb, mx=True)


@pytest.mark.parametrize("mx", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_gemm_empty_k(nv, mx, dtype):
    """K == 0: every output is an empty sum, so the whole (strided) window of C becomes 0 and
    nothing around it changes; the operands' code and scale pointers are null and never read."""
    M, N = 300, 520
    layout = nv.MX_1x32 if mx else nv.BLK_1x16
    qa, qb = nv.QTensor.empty(M, 0, layout, DEV), nv.QTensor.empty(N, 0, layout, DEV)
    assert qa.codes.data_ptr() == 0 and qb.scales.data_ptr() == 0
    if not mx:
        qa.s_dec.fill_(1.0)
        qb.s_dec.fill_(1.0)
    big = torch.full((M, N + 40), 7.0, dtype=dtype, device=DEV)
    out = big[:, 8:8 + N]
    (nv.mx_gemm if mx else nv.gemm)(qa, qb, dtype, out=out)
    torch.cuda.synchronize()
    host = big.cpu().float()
    assert torch.all(host[:, 8:8 + N] == 0)
    assert torch.all(host[:, :8] == 7) and torch.all(host[:, 8 + N:] == 7)
