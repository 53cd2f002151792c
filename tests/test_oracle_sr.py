"""Pins for the oracle's stochastic rounding: unbiasedness over many seeds, the exact round-up
probability, outputs restricted to the two neighbours, and fixed points."""
import numpy as np
import pytest
import torch

import workloads as W

GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _val(code):
    m = GRID[code & 7]
    return np.where(code & 8, -m, m)


@pytest.mark.parametrize("z", [0.3, 0.7, 1.1, 1.9, 2.7, 3.2, 4.9, 5.99, -0.45, -3.3])
def test_sr_is_unbiased_over_seeds(orc, z):
    n = 100000
    seeds = np.arange(n, dtype=np.uint64)
    # one element (index 13) under n different seeds
    r16 = np.array([orc.sr_bits(int(s), 13) for s in seeds[:20000]] +
                   list(orc.sr_bits_n(123457, np.arange(n - 20000, dtype=np.uint64) * 8 + 5)),
                   dtype=np.uint32)
    codes = orc.e2m1_sr_n(np.full(n, z, dtype=np.float32), r16)
    v = _val(codes)
    a = abs(np.float32(z))
    lo = GRID[GRID <= a].max()
    hi = GRID[GRID > a].min()
    assert set(np.unique(np.abs(v))) <= {lo, hi}
    p = (a - lo) / (hi - lo)
    sigma = (hi - lo) * np.sqrt(p * (1 - p) / n)
    assert abs(v.mean() - np.float32(z)) < 5 * sigma + 1e-12
    # the round-up probability is exactly ceil(65536 p) / 65536 for a 16-bit uniform
    ups = int((np.abs(v) == hi).sum())
    pe = np.ceil(65536 * p) / 65536
    assert abs(ups - n * pe) < 5 * np.sqrt(n * pe * (1 - pe))


def test_sr_threshold_is_exact(orc):
    # p = 0.25 exactly for z = 0.125 between 0 and 0.5: r16 < 16384 rounds up
    assert orc.e2m1_sr(0.125, 16383) == 1 and orc.e2m1_sr(0.125, 16384) == 0
    # grid points never move
    for c in range(16):
        for r in (0, 1, 32768, 65535):
            assert orc.e2m1_sr(float(_val(np.uint8(c))), r) == c
    # beyond the largest magnitude: saturate without randomness
    assert orc.e2m1_sr(7.5, 0) == 7 and orc.e2m1_sr(-1e9, 65535) == 15


def test_sr_quantizer_unbiased_over_seeds(orc):
    """Mean of the dequantized SR tensor over many seeds approaches the input (block scales are
    deterministic, only the element rounding is random)."""
    x = W.grad((4, 64), 301)
    xb = W.bits(x)
    n = 3000
    acc = np.zeros(x.shape)
    acc2 = np.zeros(x.shape)
    for s in range(n):
        q = orc.quantize_1d(xb, rounding=1, seed=s)
        xh = orc.dequantize(q, *x.shape).astype(np.float64)
        acc += xh
        acc2 += xh * xh
    mean = acc / n
    var = np.maximum(acc2 / n - mean ** 2, 0)
    xf = x.to(torch.float64).numpy()
    rnd = var > 0
    tol = 5 * np.sqrt(var / n) + 1e-6 * np.abs(xf).max()
    assert rnd.sum() > 100
    assert np.all(np.abs(mean - xf)[rnd] <= tol[rnd])
    # elements that never moved are grid points or saturated at the block maximum (|z| > 6,
    # possible when the E4M3 block scale rounded below its target)
    q = orc.quantize_1d(xb, rounding=1, seed=0)
    s = torch.from_numpy(q["scales"]).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    top = 6 * np.repeat(s, 16, axis=1) * q["s_dec"]
    fixed = ~rnd
    assert np.all((np.abs(mean - xf) <= 1e-6 * np.abs(xf).max())[fixed] |
                  (np.isclose(np.abs(mean), top, rtol=1e-6) & (np.abs(xf) >= np.abs(mean)))[fixed])


def test_sr_reproducible_and_seed_dependent(orc):
    x = W.grad((16, 128), 7)
    xb = W.bits(x)
    a = orc.quantize_1d(xb, rounding=1, seed=42)
    b = orc.quantize_1d(xb, rounding=1, seed=42)
    c = orc.quantize_1d(xb, rounding=1, seed=43)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    assert not np.array_equal(a["codes"], c["codes"])
    np.testing.assert_array_equal(a["scales"], c["scales"])
