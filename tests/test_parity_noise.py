"""GPU parity of the quantizer's fused quantization-noise diagnostic: codes and scales bit-exact
against the oracle's 1D quantization, the two sums (sum x^2, sum (Q(x) - x)^2) within a relative
1e-5 of the oracle's float64 sums (the GPU accumulates 16-element blocks in fp32 and
combines them in fp64 in a run-dependent order)."""
import numpy as np
import pytest
import torch

import workloads as W
from nvfp4_bit_quantized_amd.diagnostics import noise_report as _noise_report

pytestmark = pytest.mark.gpu

DEV = "cuda"
REL = 1e-5


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _check(nv, orc, x, rounding, seed):
    q, sums = nv.quantize_1d_noise(x.to(DEV), rounding, seed)
    torch.cuda.synchronize()
    xb = W.bits(x)
    o = orc.quantize_1d(xb, rounding=rounding, seed=seed)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), o["codes"])
    np.testing.assert_array_equal(q.scales.cpu().numpy(), o["scales"])
    g2, e2 = orc.quant_noise(xb, o)
    got = sums.cpu().numpy()
    assert abs(got[0] - g2) <= REL * g2, (got, g2)
    assert abs(got[1] - e2) <= REL * e2, (got, e2)
    return got, (g2, e2)


SMALL = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
         ("bf16_ragged", lambda: W.act((37, 80), 5)),
         ("bf16_grad", lambda: W.grad((64, 4096 + 48), 7))]


@pytest.mark.parametrize("name,make", SMALL)
@pytest.mark.parametrize("rounding", [0, 1])
def test_noise_small(nv, orc, name, make, rounding):
    _check(nv, orc, make(), rounding, 0x77)


def test_noise_hand_worked_tensor(nv):
    # block 0 decodes exactly, block 1 has three midpoint elements with errors 0.5, 1 and 0.25
    b0 = [10.5, -10.5, 0.0, 0.875, 1.75, -2.625, 3.5, 5.25, 7.0, -7.0] + [0.0] * 6
    b1 = [6.0, 2.5, 5.0, 0.25] + [0.0] * 12
    x = torch.tensor([b0 + b1], dtype=torch.bfloat16, device=DEV)
    for rounding in (0, 1):
        _, sums = nv.quantize_1d_noise(x, rounding, 5)
        got = sums.cpu().tolist()
        assert abs(got[0] - 436.34375) <= 1e-9 and abs(got[1] - 1.3125) <= 1e-9, got


def test_noise_sums_are_overwritten(nv):
    x = W.grad((64, 256), 9).to(DEV)
    sums = torch.full((2,), 123.0, dtype=torch.float64, device=DEV)
    _, a = nv.quantize_1d_noise(x, 1, 3, sums=sums)
    first = a.cpu().tolist()
    _, b = nv.quantize_1d_noise(x, 1, 3, sums=sums)
    second = b.cpu().tolist()
    assert abs(first[0] - second[0]) <= 1e-12 * first[0]
    assert abs(first[1] - second[1]) <= 1e-12 * first[1]


def test_noise_full_size_dgrad_operand(nv, orc):
    """dY 8192 x 4096 with SR at the dgrad seed: whole-tensor sums against the oracle."""
    x = W.grad((8192, 4096), W.CFG3["seed"])
    got, ref = _check(nv, orc, x, 1, W.CFG3["sr_seed"])
    rep = _noise_report(torch.tensor(got))
    assert rep["ratio"] == pytest.approx((ref[0] / ref[1]) ** 0.5, rel=1e-5)


def _check_rht(nv, orc, x, rounding, seed, sign_seed):
    """The Hadamard quantizer's noise sums against the oracle's on the transformed tensor."""
    q, sums = nv.hadamard_quantize_noise(x.to(DEV), sign_seed, rounding, seed)
    torch.cuda.synchronize()
    xb = W.bits(x)
    o = orc.hadamard_quantize(xb, sign_seed, rounding=rounding, seed=seed)
    np.testing.assert_array_equal(q.codes.cpu().numpy(), o["codes"])
    np.testing.assert_array_equal(q.scales.cpu().numpy(), o["scales"])
    g2, e2 = orc.quant_noise(orc.hadamard_transform(xb, sign_seed), o)
    got = sums.cpu().numpy()
    assert abs(got[0] - g2) <= REL * g2, (got, g2)
    assert abs(got[1] - e2) <= REL * e2, (got, e2)
    return got, (g2, e2)


@pytest.mark.parametrize("rounding", [0, 1])
@pytest.mark.parametrize("T,F", [(64, 24), (512, 64), (528, 136)])
def test_hadamard_noise_small(nv, orc, rounding, T, F):
    _check_rht(nv, orc, W.grad((T, F), T + F), rounding, 0x99, 0x51E4)


def test_hadamard_noise_full_size_wgrad_operand(nv, orc):
    """dY 16384 x 4096 through the Hadamard quantizer with SR at the wgrad seeds (the capped
    grid takes two chunk blocks per workgroup here): whole-tensor sums against the oracle, and
    the transformed tensor's squared norm equals the input's to rounding (orthogonal transform)."""
    x = W.grad((16384, 4096), W.CFG4["seeds"][1])
    got, ref = _check_rht(nv, orc, x, 1, W.CFG4["sr_seed"], W.CFG4["sign_seed"])
    xv = orc.values(W.bits(x))
    assert got[0] == pytest.approx(float(np.sum(xv * xv)), rel=1e-5)
