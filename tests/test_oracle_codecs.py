"""Pins for the oracle's scalar codecs: E2M1, E4M3, Philox4x32-10, bf16 rounding.

Each check compares the oracle with something other than itself: the value set printed on the
pages, an independent rounding formulation, a library routine (torch's float8_e4m3fn and bf16
casts), or published known-answer vectors.
"""
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_e2m1_magnitudes():
    vals = []
    with open(os.path.join(GOLDEN, "e2m1_value_set.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(float(line))
    return vals


# ---- E2M1 ---------------------------------------------------------------------------------------
def test_e2m1_decode_matches_printed_value_set(orc):
    mags = _page_e2m1_magnitudes()
    assert len(mags) == 8                        # 3 magnitude bits
    got = [orc.e2m1_value(c) for c in range(16)]
    # codes 0..7 are the positive values in increasing order, 8..15 their negatives
    assert got[:8] == mags
    assert [-v for v in mags] == got[8:]
    assert np.signbit(got[8]) and not np.signbit(got[0])


def _minifloat_round(a: np.ndarray) -> np.ndarray:
    """Generic IEEE-style round-to-nearest-even of |z| onto a 1-mantissa-bit, 2-exponent-bit
    format with bias 1 and saturation at its largest value 6: the quantum in binade E >= 0 is
    2^(E-1) and numpy's round() breaks ties to the even multiple."""
    a = a.astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 1e-300)))
    e = np.clip(e, 0, None)                      # below 1.0 the subnormal quantum 0.5 applies
    q = np.exp2(e - 1)
    r = np.round(a / q) * q
    return np.minimum(r, 6.0)


def _e2m1_index(values: np.ndarray) -> np.ndarray:
    mags = np.array(_page_e2m1_magnitudes())
    idx = np.searchsorted(mags, values)
    assert np.all(mags[idx] == values)
    return idx


def test_e2m1_rne_matches_generic_minifloat_rounding(orc):
    # every fp32 in [0, 16] whose low 11 mantissa bits are zero, plus both neighbours of every
    # tie point, plus random fp32 in [0, 10]
    bits = np.arange(0, 0x41800000, 1 << 11, dtype=np.uint64).astype(np.uint32)
    z = bits.view(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    near = np.concatenate([ties, np.nextafter(ties, np.float32(0)), np.nextafter(ties, np.float32(10))])
    rng = np.random.default_rng(7)
    z = np.concatenate([z, near, rng.uniform(0, 10, 200000).astype(np.float32)])
    codes = orc.e2m1_rne_n(z)
    expect = _e2m1_index(_minifloat_round(z))
    np.testing.assert_array_equal(codes, expect)
    # negative inputs: same magnitude code with the sign bit
    np.testing.assert_array_equal(orc.e2m1_rne_n(-z), expect | 8)


def test_e2m1_rne_tie_table_and_sign(orc):
    # halfway points go to the even code (mantissa bit 0)
    table = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             6.0: 6.0, 7.0: 6.0, 1e30: 6.0}
    for z, v in table.items():
        assert orc.e2m1_value(orc.e2m1_rne(z)) == v, z
    assert orc.e2m1_rne(-0.0) == 0x8               # signed zero kept
    assert orc.e2m1_rne(-0.1) == 0x8               # negative value rounding to zero
    assert orc.e2m1_rne(-100.0) == 0xF
    for c in range(16):                            # grid points are fixed points
        assert orc.e2m1_rne(orc.e2m1_value(c)) == c


# ---- E4M3 ---------------------------------------------------------------------------------------
def test_e4m3_decode_matches_torch(orc):
    b = torch.arange(0, 0x7F, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_value(int(i)) for i in range(0x7F)])
    np.testing.assert_array_equal(got, ref)
    assert got[0x7E] == 448.0
    assert np.isnan(orc.e4m3_value(0x7F))


def test_e4m3_encode_matches_torch_cast(orc):
    rng = np.random.default_rng(11)
    vals = [np.arange(0, 0x43E80000, 1 << 13, dtype=np.uint64).astype(np.uint32).view(np.float32),
            rng.uniform(0, 470, 300000).astype(np.float32),
            np.exp2(rng.uniform(-14, 9, 300000)).astype(np.float32)]
    # every midpoint between consecutive E4M3 values, and its fp32 neighbours
    grid = np.array([orc.e4m3_value(i) for i in range(0x7F)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e4))]
    t = np.concatenate(vals)
    got = orc.e4m3_rne_sat_n(t)
    ref = torch.from_numpy(np.minimum(t, np.float32(448.0))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    assert orc.e4m3_rne_sat(464.0) == 0x7E and orc.e4m3_rne_sat(1e30) == 0x7E
    # spot values: ties to the even byte
    assert orc.e4m3_value(orc.e4m3_rne_sat(1.0625)) == 1.0
    assert orc.e4m3_value(orc.e4m3_rne_sat(1.1875)) == 1.25
    assert orc.e4m3_value(orc.e4m3_rne_sat(17.0)) == 16.0
    assert orc.e4m3_value(orc.e4m3_rne_sat(19.0)) == 20.0
    assert orc.e4m3_rne_sat(2.0 ** -10) == 0


# ---- Philox4x32-10 ------------------------------------------------------------------------------
def test_philox_known_answers(orc):
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            ctr, key, out = w[0:4], w[4:6], w[6:10]
            np.testing.assert_array_equal(orc.philox4x32_10(ctr, key), np.array(out, dtype=np.uint32))
            n += 1
    assert n == 3


def test_sr_bits_are_uniform_16bit(orc):
    idx = np.arange(1 << 18, dtype=np.uint64)
    r = orc.sr_bits_n(0x1234, idx)
    assert r.max() < 65536
    # chi-square over 64 bins, 262144 draws: far inside any plausible acceptance region
    h = np.bincount(r >> 10, minlength=64)
    e = len(r) / 64
    chi2 = ((h - e) ** 2 / e).sum()
    assert chi2 < 140, chi2
    # the eight elements of a counter draw from four distinct words
    w = orc.philox4x32_10([5, 0, 0, 0], [0x1234, 0])
    exp = [w[0] & 0xFFFF, w[0] >> 16, w[1] & 0xFFFF, w[1] >> 16, w[2] & 0xFFFF, w[2] >> 16,
           w[3] & 0xFFFF, w[3] >> 16]
    assert [orc.sr_bits(0x1234, 40 + i) for i in range(8)] == exp


# ---- bf16 rounding ------------------------------------------------------------------------------
def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.integers(0, 1 << 31, 20000, dtype=np.uint32)).view(np.float32)])
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.f32_to_bf16(float(v)) for v in x], dtype=np.uint16)
    ok = np.abs(x) < 3.0e38        # skip values that round to inf
    np.testing.assert_array_equal(got[ok], ref[ok])


def test_tensor_scales(orc):
    k1, s_enc, s_dec = orc.tensor_scales(3.0)
    assert k1 == np.float32(448.0) / np.float32(3.0)
    assert s_enc == np.float32(2688.0) / np.float32(3.0)
    assert s_dec == np.float32(3.0) / np.float32(2688.0)
    assert orc.tensor_scales(0.0) == (448.0, 1.0, 1.0)
