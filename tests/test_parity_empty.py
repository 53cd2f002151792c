"""Empty tensors through every entry point: nothing is read (the data pointers are null), calls
return success, and the per-tensor scalars take their zero-tensor values (amax 0, and s_dec 1
since an amax below 2^-100 counts as zero); an empty GEMM output stays empty.  (A GEMM with an
empty inner dimension, which writes zeros, is tested with the GEMMs.)"""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _scalars(q):
    torch.cuda.synchronize()
    return q.amax.item(), q.s_dec.item()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_quantizers(nv, dtype):
    e_rows = torch.empty((0, 64), dtype=dtype, device=DEV)      # no rows
    e_cols = torch.empty((32, 0), dtype=dtype, device=DEV)      # no columns
    e_tok = torch.empty((0, 16), dtype=dtype, device=DEV)       # no tokens
    assert e_rows.data_ptr() == 0 and e_tok.data_ptr() == 0
    for x in (e_rows, e_cols):
        a = nv.amax(x)
        torch.cuda.synchronize()
        assert a.item() == 0.0
        for rnd in (nv.RNE, nv.SR):
            assert _scalars(nv.quantize_1d(x, rnd, 5)) == (0.0, 1.0)
        q, _ = nv.quantize_1d_noise(x, nv.SR, 5)
        assert _scalars(q) == (0.0, 1.0)
        nv.mx_quantize_1d(x)
        y = nv.dequantize(nv.quantize_1d(x), dtype)
        assert y.shape == x.shape
    q, qt = nv.quantize_2d(torch.empty((0, 32), dtype=dtype, device=DEV), transposed=True)
    assert _scalars(q) == (0.0, 1.0) and _scalars(qt) == (0.0, 1.0)
    torch.cuda.synchronize()
    assert nv.hadamard_amax(e_tok, 7).item() == 0.0
    for rnd in (nv.RNE, nv.SR):
        assert _scalars(nv.hadamard_quantize(e_tok, 7, rnd, 3)) == (0.0, 1.0)
        r, t = nv.quantize_dual(e_tok, 7, rnd, 3, 4)
        assert _scalars(r) == (0.0, 1.0) and _scalars(t) == (0.0, 1.0)
        qn, sums = nv.hadamard_quantize_noise(e_tok, 7, rnd, 3)
        assert _scalars(qn) == (0.0, 1.0) and sums.cpu().tolist() == [0.0, 0.0]
    nv.mx_quantize_1d_t(torch.empty((0, 32), dtype=dtype, device=DEV))
    torch.cuda.synchronize()


@pytest.mark.parametrize("mx", [False, True])
def test_empty_gemm_outputs(nv, mx):
    K = 256
    layout = nv.MX_1x32 if mx else nv.BLK_1x16
    full = nv.QTensor.empty(64, K, layout, DEV)
    full.codes.zero_()
    full.scales.fill_(0x7F if mx else 0x38)
    if not mx:
        full.s_dec.fill_(1.0)
    none = nv.QTensor.empty(0, K, layout, DEV)
    if not mx:
        none.s_dec.fill_(1.0)
    gemm = nv.mx_gemm if mx else nv.gemm
    for dtype in (torch.float32, torch.bfloat16):
        assert gemm(none, full, dtype).shape == (0, 64)
        assert gemm(full, none, dtype).shape == (64, 0)
    torch.cuda.synchronize()
