"""Pins of the oracle's format-sweep quantizer (block size 8 / 16 / 32, E4M3 or E8M0 scales, RNE
or SR; "FP4 All the Way", Describir: block size, scale format and rounding are the FP4 design
choices explored, and 16-element blocks with E4M3 scales come out best).  The special cases
reduce to the already pinned NVFP4 and MXFP4 quantizers; the others are worked by hand."""
import numpy as np
import pytest
import torch

import workloads as W


@pytest.mark.parametrize("rounding", [0, 1])
def test_block16_e4m3_is_nvfp4(orc, rounding):
    x = W.grad((64, 256), 31)
    xb = W.bits(x)
    y, A = orc.qdq(xb, 16, 0, rounding, 9)
    q = orc.quantize_1d(xb, rounding=rounding, seed=9)
    np.testing.assert_array_equal(y, orc.dequantize(q, 64, 256))
    assert A == q["amax"]


@pytest.mark.parametrize("rounding", [0, 1])
def test_block32_e8m0_is_mxfp4(orc, rounding):
    x = W.act((48, 256), 32)
    xb = W.bits(x)
    y, A = orc.qdq(xb, 32, 1, rounding, 10)
    q = orc.mx_quantize_1d(xb, rounding=rounding, seed=10)
    np.testing.assert_array_equal(y, orc.mx_dequantize(q, 48, 256))
    assert A == 0.0


def test_e8m0_clips_the_block_maximum_e4m3_does_not(orc):
    # block [7, 1, 0 ...]: E8M0 takes 2^(floor(log2 7) - 2) = 1, so 7 saturates to 6 (error 1);
    # with E4M3 and the tensor scale the block maximum maps to 6 * scale = 7 up to rounding
    x = np.zeros((1, 8), dtype=np.float32)
    x[0, 0], x[0, 1] = 7.0, 1.0
    y8, _ = orc.qdq(x, 8, 1)
    assert y8[0, 0] == 6.0 and y8[0, 1] == 1.0
    y4, A = orc.qdq(x, 8, 0)
    assert A == 7.0 and abs(y4[0, 0] - 7.0) <= 7.0 * 2 ** -20


def test_block8_halves_share_no_scale(orc):
    # two 8-element blocks of very different magnitude: each gets its own E8M0 scale, so the small
    # block is exact (values on its grid) although a 16-block would have flushed it
    x = np.zeros((1, 16), dtype=np.float32)
    x[0, :8] = [6.0, -4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.0]
    x[0, 8:] = np.array([6.0, -4.0, 3.0, 2.0, 1.5, 1.0, 0.5, 0.0]) * 2.0 ** -10
    y8, _ = orc.qdq(x, 8, 1)
    np.testing.assert_array_equal(y8, x)
    y16, _ = orc.qdq(x, 16, 1)
    np.testing.assert_array_equal(y16[0, :8], x[0, :8])
    assert np.all(y16[0, 8:] == 0.0)
