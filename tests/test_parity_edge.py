"""GPU parity at the edges of the formats' ranges (the degenerate cases of the method), fp32
inputs from workloads.edge_fp32: fp32 subnormals with the tensor amax below the 2^-100 zero
threshold, an amax just above it, an amax near the top of the fp32 range, blocks whose E4M3 scale
is subnormal or zero next to large blocks, signed zeros, subnormal values beside normal ones, and
Hadamard-transformed amaxes just below and above 2^120; the same tensors in bf16 through the
Hadamard, dual and MXFP4 dual quantizers (whose bf16 path folds the transform's 1/4 into the
encode factor while the amax is at most 2^120, for both roundings).  Every quantizer's codes, scale
bytes, amax and s_dec must equal the oracle's bit for bit; dequantized values exactly; a GEMM of
each tensor with a normal weight within relative L2 1e-5."""
import numpy as np
import pytest
import torch

import workloads as W
from gemm_check import assert_gemm_close

pytestmark = pytest.mark.gpu

DEV = "cuda"
KINDS = ["tiny", "near_zero", "huge", "wide", "signed_zeros", "tiny_mix", "below_2p120", "above_2p120"]
SIGN = 0x51E40006


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _np(t):
    return t.cpu().numpy()


def _same_q(g, o, what, scalars=True):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(g.codes), o["codes"], err_msg=f"codes {what}")
    np.testing.assert_array_equal(_np(g.scales), o["scales"], err_msg=f"scales {what}")
    if scalars:
        assert float(g.amax.item()) == o["amax"], what
        assert float(g.s_dec.item()) == o["s_dec"], what


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rounding", [0, 1])
def test_edge_1d_and_dequantize(nv, orc, kind, rounding):
    x = W.edge_fp32(kind, (64, 96), 41)
    xb = W.bits(x)
    g = nv.quantize_1d(x.to(DEV), rounding, seed=0x5EED0041)
    o = orc.quantize_1d(xb, rounding, 0x5EED0041)
    _same_q(g, o, f"1d {kind}")
    np.testing.assert_array_equal(_np(nv.dequantize(g)), orc.dequantize(o, 64, 96))


@pytest.mark.parametrize("kind", KINDS)
def test_edge_2d(nv, orc, kind):
    w = W.edge_fp32(kind, (48, 64), 42)
    g, gt = nv.quantize_2d(w.to(DEV), transposed=True)
    o = orc.quantize_2d(W.bits(w))
    _same_q(g, o, f"2d {kind}")
    np.testing.assert_array_equal(_np(gt.codes), o["codes_t"])
    np.testing.assert_array_equal(_np(gt.scales), o["scales_t"])


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rounding", [0, 1])
def test_edge_hadamard(nv, orc, kind, rounding):
    x = W.edge_fp32(kind, (64, 48), 43)
    xb = W.bits(x)
    g = nv.hadamard_quantize(x.to(DEV), SIGN, rounding, seed=7)
    _same_q(g, orc.hadamard_quantize(xb, SIGN, rounding, 7), f"rht {kind}")
    q, qt = nv.quantize_dual(x.to(DEV), SIGN, rounding, seed=8, seed_t=9)
    _same_q(q, orc.quantize_1d(xb, rounding, 8), f"dual rows {kind}")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, rounding, 9), f"dual transposed {kind}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rounding", [0, 1])
def test_edge_mx(nv, orc, kind, rounding):
    x = W.edge_fp32(kind, (64, 96), 44)
    xb = W.bits(x)
    g = nv.mx_quantize_1d(x.to(DEV), rounding, seed=10)
    o = orc.mx_quantize_1d(xb, rounding, 10)
    _same_q(g, o, f"mx {kind}", scalars=False)
    np.testing.assert_array_equal(_np(nv.dequantize(g)), orc.mx_dequantize(o, 64, 96))
    gt = nv.mx_quantize_1d_t(x.to(DEV), rounding, seed=11)
    _same_q(gt, orc.mx_quantize_1d(np.ascontiguousarray(xb.T), rounding, 11), f"mx_t {kind}",
            scalars=False)


@pytest.mark.parametrize("kind", KINDS)
def test_edge_gemm(nv, orc, kind):
    a = W.edge_fp32(kind, (64, 64), 45)
    b = W.weight((32, 64), 46).float()
    qa, qb = nv.quantize_1d(a.to(DEV)), nv.quantize_1d(b.to(DEV))
    c = nv.gemm(qa, qb, torch.float32)
    torch.cuda.synchronize()
    oa, ob = orc.quantize_1d(W.bits(a)), orc.quantize_1d(W.bits(b))
    ref = orc.gemm_f64(oa, ob, 64, 32, 64)
    got = _np(c).astype(np.float64)
    den = np.linalg.norm(ref)
    if den == 0.0:
        assert not got.any()
    else:
        assert_gemm_close(got, ref, "edge gemm")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rounding", [0, 1])
def test_edge_bf16_hadamard_and_dual(nv, orc, kind, rounding):
    x = W.edge_fp32(kind, (64, 48), 47, torch.bfloat16)
    xb = W.bits(x)
    g = nv.hadamard_quantize(x.to(DEV), SIGN, rounding, seed=12)
    _same_q(g, orc.hadamard_quantize(xb, SIGN, rounding, 12), f"bf16 rht {kind}")
    q, qt = nv.quantize_dual(x.to(DEV), SIGN, rounding, seed=13, seed_t=14)
    _same_q(q, orc.quantize_1d(xb, rounding, 13), f"bf16 dual rows {kind}")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, rounding, 14), f"bf16 dual transposed {kind}")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("rounding", [0, 1])
def test_edge_bf16_mx_dual(nv, orc, kind, rounding):
    x = W.edge_fp32(kind, (64, 64), 48, torch.bfloat16)
    xb = W.bits(x)
    q, qt = nv.mx_quantize_dual(x.to(DEV), rounding, seed=15, seed_t=16)
    _same_q(q, orc.mx_quantize_1d(xb, rounding, 15), f"bf16 mx dual rows {kind}", scalars=False)
    _same_q(qt, orc.mx_quantize_1d(np.ascontiguousarray(xb.T), rounding, 16),
            f"bf16 mx dual transposed {kind}", scalars=False)
