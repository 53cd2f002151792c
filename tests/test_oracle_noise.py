"""Pins of the oracle's quantization-noise diagnostic (sum x^2, sum (Q(x) - x)^2), from "FP4 All
the Way" (Describir: quantized training loses efficiency once the gradient norm falls below
about sqrt(3) times the quantization noise).  The expected values are worked out by hand from
the format's rounding rules, not by the oracle."""
import numpy as np
import pytest
import torch

import workloads as W


def _pin_tensor():
    """Two NVFP4 blocks in bf16, tensor amax A = 10.5 (so s_enc = 2688 / A = 256, s_dec = 2^-8).

    Block 0 holds +-10.5, so its E4M3 scale is 448 and its elements v * 1.75 (v on the E2M1 grid)
    encode to v exactly: no error.  Block 1 has amax 6, scale 256, encode factor 256 / 256 = 1, so
    z = x: 6 is exact, and 2.5, 5 and 0.25 sit exactly midway between grid points (2|3, 4|6,
    0|0.5).  Round-to-nearest-even takes the even code (2, 4, 0); stochastic rounding takes either
    neighbour, and both are the same distance away.  The errors are 0.5, 1 and 0.25 either way."""
    b0 = [10.5, -10.5, 0.0, 0.875, 1.75, -2.625, 3.5, 5.25, 7.0, -7.0] + [0.0] * 6
    b1 = [6.0, 2.5, 5.0, 0.25] + [0.0] * 12
    x = torch.tensor([b0 + b1], dtype=torch.bfloat16)
    g2 = sum(v * v for v in b0 + b1)
    e2 = 0.5 ** 2 + 1.0 ** 2 + 0.25 ** 2
    return x, g2, e2


@pytest.mark.parametrize("rounding", [0, 1])
def test_noise_of_midpoints_is_known(orc, rounding):
    x, g2, e2 = _pin_tensor()
    xb = W.bits(x)
    q = orc.quantize_1d(xb, rounding=rounding, seed=99)
    assert q["amax"] == 10.5 and q["s_dec"] == 2.0 ** -8
    assert list(q["scales"][0]) == [0x7E, 0x78]        # E4M3 448 and 256
    got = orc.quant_noise(xb, q)
    assert got == (g2, e2) == (436.34375, 1.3125)


def test_lossless_tensor_has_zero_noise(orc):
    # every block holds +-A with A = 2688 * 2^-8, all values v * 1.75: each block decodes exactly
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6]) * 1.75
    rng = np.random.default_rng(5)
    vals = rng.choice(grid, size=(8, 64)) * rng.choice([-1.0, 1.0], size=(8, 64))
    vals[:, ::16] = 10.5
    x = torch.tensor(vals, dtype=torch.bfloat16)
    q = orc.quantize_1d(W.bits(x))
    g2, e2 = orc.quant_noise(W.bits(x), q)
    assert e2 == 0.0
    assert g2 == float(np.sum(vals.astype(np.float64) ** 2))


def test_noise_scales_with_the_tensor(orc):
    # multiplying x by 2^k scales every decoded value by 2^k exactly (amax, s_dec and the codes
    # follow), so the sums scale by 4^k
    x = W.grad((32, 128), 3).float()
    q1 = orc.quantize_1d(W.bits(x), rounding=1, seed=4)
    x8 = x * 8.0
    q8 = orc.quantize_1d(W.bits(x8), rounding=1, seed=4)
    np.testing.assert_array_equal(q1["codes"], q8["codes"])
    a = orc.quant_noise(W.bits(x), q1)
    b = orc.quant_noise(W.bits(x8), q8)
    assert b == (a[0] * 64.0, a[1] * 64.0)
