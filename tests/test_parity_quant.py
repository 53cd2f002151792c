"""GPU parity of the quantizers, amax and dequantize against the CPU oracle: bit-exact codes,
scale bytes, amax and s_dec, at small ragged sizes and at the full workload sizes."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _host(t):
    return t.detach().cpu().numpy()


def _same_q(gq, oq, what=""):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(gq.codes), oq["codes"], err_msg=f"codes {what}")
    np.testing.assert_array_equal(_host(gq.scales), oq["scales"], err_msg=f"scales {what}")
    assert float(gq.amax.item()) == oq["amax"], what
    assert float(gq.s_dec.item()) == oq["s_dec"], what


SMALL = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
         ("bf16_ragged", lambda: W.act((37, 80), 5)),
         ("bf16_one_row", lambda: W.grad((1, 16), 6)),
         ("bf16_wide", lambda: W.act((3, 4096 + 48), 7))]


@pytest.mark.parametrize("name,make", SMALL)
def test_amax_small(nv, orc, name, make):
    x = make()
    got = nv.amax(x.to(DEV))
    assert float(got.item()) == orc.amax(W.bits(x))


@pytest.mark.parametrize("name,make", SMALL)
@pytest.mark.parametrize("rounding", [0, 1])
def test_quantize_1d_small(nv, orc, name, make, rounding):
    x = make()
    g = nv.quantize_1d(x.to(DEV), rounding=rounding, seed=0x1234)
    _same_q(g, orc.quantize_1d(W.bits(x), rounding=rounding, seed=0x1234), name)


def test_quantize_1d_strided_and_supplied_amax(nv, orc):
    big = W.act((64, 160), 9)
    x = big[:, 16:16 + 128]                                   # ld = 160, offset 16 elements
    g = nv.quantize_1d(big.to(DEV)[:, 16:16 + 128], seed=3)
    _same_q(g, orc.quantize_1d(W.bits(x.contiguous())), "strided")
    a = torch.tensor([3.5], dtype=torch.float32, device=DEV)
    g = nv.quantize_1d(big.to(DEV)[:, 16:16 + 128], amax_in=a, rounding=1, seed=11)
    _same_q(g, orc.quantize_1d(W.bits(x.contiguous()), rounding=1, seed=11, amax_in=3.5), "amax_in")


def test_quantize_1d_empty_and_zero(nv, orc):
    g = nv.quantize_1d(torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert g.amax.item() == 0.0 and g.s_dec.item() == 1.0
    z = torch.zeros((4, 64), dtype=torch.bfloat16)
    z[1, 3] = -0.0
    _same_q(nv.quantize_1d(z.to(DEV)), orc.quantize_1d(W.bits(z)), "zeros")


def test_quantize_1d_sr_deterministic_and_seeded(nv):
    x = W.grad((64, 512), 12).to(DEV)
    a = nv.quantize_1d(x, rounding=1, seed=77)
    b = nv.quantize_1d(x, rounding=1, seed=77)
    c = nv.quantize_1d(x, rounding=1, seed=78)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes)
    assert not torch.equal(a.codes, c.codes)


@pytest.mark.parametrize("name,make", [("w_ragged", lambda: W.weight((48, 80), 21)),
                                       ("w_fp32", lambda: W.small_fp32((64, 32), 22)),
                                       ("w_rect", lambda: W.weight((160, 96), 23)),
                                       # several 128x128 workgroup regions in both dimensions,
                                       # with 16-wide tails
                                       ("w_regions", lambda: W.weight((272, 400), 24)),
                                       ("w_regions_fp32", lambda: W.small_fp32((400, 272), 25))])
def test_quantize_2d_small(nv, orc, name, make):
    w = make()
    g, gt = nv.quantize_2d(w.to(DEV), transposed=True)
    o = orc.quantize_2d(W.bits(w))
    _same_q(g, o, name)
    np.testing.assert_array_equal(_host(gt.codes), o["codes_t"])
    np.testing.assert_array_equal(_host(gt.scales), o["scales_t"])
    assert gt.s_dec.item() == o["s_dec"]


def test_quantize_2d_strided(nv, orc):
    """A weight that is a column slice of a wider matrix (row stride > cols)."""
    big = W.weight((144, 320), 26)
    w = big[:, 48:48 + 256]
    g, gt = nv.quantize_2d(big.to(DEV)[:, 48:48 + 256], transposed=True)
    o = orc.quantize_2d(W.bits(w.contiguous()))
    _same_q(g, o, "strided")
    np.testing.assert_array_equal(_host(gt.codes), o["codes_t"])
    np.testing.assert_array_equal(_host(gt.scales), o["scales_t"])


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("T,F", [(48, 24), (512, 64), (528, 136), (640, 264)])
def test_hadamard_quantize_small(nv, orc, rounding, T, F):
    x = W.act((T, F), T + F)
    g = nv.hadamard_quantize(x.to(DEV), sign_seed=0x51E4, rounding=rounding, seed=5)
    _same_q(g, orc.hadamard_quantize(W.bits(x), 0x51E4, rounding=rounding, seed=5), f"rht {T}x{F}")
    ga = nv.hadamard_amax(x.to(DEV), 0x51E4)
    assert ga.item() == orc.hadamard_amax(W.bits(x), 0x51E4)


@pytest.mark.parametrize("layout", ["1d", "2d"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize(nv, orc, layout, dtype):
    x = W.act((64, 96), 31)
    if layout == "1d":
        g = nv.quantize_1d(x.to(DEV))
        o = orc.quantize_1d(W.bits(x))
    else:
        g, _ = nv.quantize_2d(x.to(DEV), transposed=False)
        o = orc.quantize_2d(W.bits(x), transposed=False)
    y = nv.dequantize(g, dtype)
    ref = orc.dequantize(o, 64, 96, out_bf16=(dtype == torch.bfloat16))
    torch.cuda.synchronize()
    if dtype == torch.bfloat16:
        np.testing.assert_array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), ref)
    else:
        np.testing.assert_array_equal(y.cpu().numpy(), ref)


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("shape", [(64, 96), (5, 4096)])
def test_mx_quantize(nv, orc, rounding, shape):
    x = W.act(shape, 41)
    g = nv.mx_quantize_1d(x.to(DEV), rounding=rounding, seed=9)
    o = orc.mx_quantize_1d(W.bits(x), rounding=rounding, seed=9)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(g.codes), o["codes"])
    np.testing.assert_array_equal(_host(g.scales), o["scales"])
    y = nv.dequantize(g)
    np.testing.assert_array_equal(y.cpu().numpy(), orc.mx_dequantize(o, *shape))


# ---- full workload sizes ------------------------------------------------------------------------
def test_full_fprop_operands(nv, orc):
    """X 8192x4096 Student-t(3) (1D, RNE) and W 4096x4096 N(0,0.02) (2D + transposed copy)."""
    x = W.act(W.CFG2["x"], W.CFG2["seeds"][0])
    g = nv.quantize_1d(x.to(DEV))
    _same_q(g, orc.quantize_1d(W.bits(x)), "X 8192x4096")
    w = W.weight(W.CFG2["w"], W.CFG2["seeds"][1])
    gw, gwt = nv.quantize_2d(w.to(DEV), transposed=True)
    o = orc.quantize_2d(W.bits(w))
    _same_q(gw, o, "W 4096x4096")
    np.testing.assert_array_equal(_host(gwt.codes), o["codes_t"])
    np.testing.assert_array_equal(_host(gwt.scales), o["scales_t"])


def test_full_dgrad_operand_sr(nv, orc):
    """dY 8192x4096 N(0,1e-3) with 0.1% x100 spikes, stochastic rounding at a fixed seed."""
    dy = W.grad(W.CFG3["dy"], W.CFG3["seed"])
    g = nv.quantize_1d(dy.to(DEV), rounding=1, seed=W.CFG3["sr_seed"])
    _same_q(g, orc.quantize_1d(W.bits(dy), rounding=1, seed=W.CFG3["sr_seed"]), "dY SR")


def test_full_wgrad_operands(nv, orc):
    """X and dY 16384x4096 through the random Hadamard transform (X RNE, dY SR)."""
    c = W.CFG4
    x = W.act(c["x"], c["seeds"][0])
    g = nv.hadamard_quantize(x.to(DEV), c["sign_seed"], rounding=0)
    _same_q(g, orc.hadamard_quantize(W.bits(x), c["sign_seed"], rounding=0), "X rht")
    del x, g
    dy = W.grad(c["dy"], c["seeds"][1])
    g = nv.hadamard_quantize(dy.to(DEV), c["sign_seed"], rounding=1, seed=c["sr_seed"])
    _same_q(g, orc.hadamard_quantize(W.bits(dy), c["sign_seed"], rounding=1, seed=c["sr_seed"]), "dY rht SR")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_full_dequantize(nv, orc, dtype):
    """Dequantize at full size, bit-exact: X 8192x4096 (1D, its codes equal the oracle's, as
    test_full_fprop_operands shows) and W 4096x4096 (16x16 tiles) to fp32 and to bf16."""
    for make, shape, seed, two_d in ((W.act, W.CFG2["x"], W.CFG2["seeds"][0], False),
                                     (W.weight, W.CFG2["w"], W.CFG2["seeds"][1], True)):
        x = make(shape, seed)
        if two_d:
            g, _ = nv.quantize_2d(x.to(DEV), transposed=False)
            o = orc.quantize_2d(W.bits(x), transposed=False)
        else:
            g = nv.quantize_1d(x.to(DEV))
            o = orc.quantize_1d(W.bits(x))
        _same_q(g, o, f"dequant operand {shape}")
        y = nv.dequantize(g, dtype)
        ref = orc.dequantize(o, *shape, out_bf16=(dtype == torch.bfloat16))
        torch.cuda.synchronize()
        got = y.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == torch.bfloat16 \
            else y.cpu().numpy()
        np.testing.assert_array_equal(got, ref, err_msg=f"dequantize {shape} {dtype}")
        del x, g, y
