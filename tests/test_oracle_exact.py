"""Pins for the two fp32 orderings the oracle fixes by reading, held against exact arithmetic.

The two-level scaling ("I ricercatori di Nvidia ...", Come funziona NVFP4?) and the block format
("Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision", Caracteristicas del Formato
NVFP4) define each block's E4M3 scale from amax_b * 448 / A and each code from
x * (2688 / A) / scale; the oracle evaluates them in fp32 in a fixed order (k1 = 448 / A,
t = ab * k1; enc = s_enc / scale, z = x * enc).  Done with exact rationals instead, the same
definitions give the same scale bytes and codes everywhere except where the exact value lies
within the few fp32 roundings of a rounding midpoint; these tests compute the exact results
here (Fractions, format value sets enumerated from their bit layouts) and allow differences
only there.  A dropped factor, a swapped scale (s_dec for s_enc, 2688 for 448), a division
for a multiplication or a wrong tie rule fails on thousands of elements.

The 16-point random Hadamard transform (same page, Metodologia de Entrenamiento) is pinned by its
matrix on integer inputs elsewhere; here the oracle's fp32 butterflies on general inputs must
stay within the rounding bound of a 4-level summation of the exact float64 product, and the
quantization of the transformed tensor must equal the exact-arithmetic quantization of the
exact transform away from midpoints.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

RNE = 0

# ---- the formats' value sets, from their bit layouts -------------------------------------------
# E2M1 magnitudes by 3-bit code: exponent field e (bias 1) and mantissa bit m; e = 0 is
# subnormal (m * 0.5).
E2M1 = [Fraction(m, 2) if e == 0 else Fraction(2 + m, 2) * 2 ** (e - 1)
        for e in range(4) for m in range(2)]
# E4M3 magnitudes by 7-bit code (0x7F is NaN, so 0..126): exponent e (bias 7), mantissa m.
E4M3 = [Fraction(m, 8) * Fraction(1, 64) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        for e in range(16) for m in range(8)][:127]
assert E2M1 == [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]
assert E4M3[-1] == 448 and E4M3[1] == Fraction(1, 512)


def rne_index(table, v: Fraction):
    """Index of the nearest entry of an increasing table to v >= 0, ties to the even index,
    saturating at the last entry; also the relative distance of v to the nearest midpoint."""
    if v >= table[-1]:
        return len(table) - 1, Fraction(1)
    lo = max(i for i, t in enumerate(table) if t <= v)
    hi = lo + 1
    mid = (table[lo] + table[hi]) / 2
    dist = abs(v - mid) / mid
    if v < mid:
        idx = lo
    elif v > mid:
        idx = hi
    else:
        idx = lo if lo % 2 == 0 else hi
    return idx, dist


def nibble(codes, r, c):
    b = int(codes[r, c // 2])
    return (b >> 4) if c & 1 else (b & 15)


# Two fp32 roundings of relative size 2^-24 each separate the oracle's scale target from the
# exact one, three its element target: a result may differ only within that distance of a
# midpoint (with a factor of 4 to spare).
TOL_SCALE = Fraction(1, 2 ** 20)
TOL_CODE = Fraction(1, 2 ** 19)


def exact_block_check(x: np.ndarray, q: dict, A_used: float, strict: bool = True):
    """Compare q (codes [R x K/2], scales [R x K/16] of x [R x K], 1x16 blocks, tensor amax
    A_used) with the exact-arithmetic definition.  Returns (elements compared, code mismatches,
    scale mismatches); strict: every mismatch must lie near a midpoint, else each must be one
    step of the format (an adjacent code or scale)."""
    rows, cols = x.shape
    A = Fraction(float(A_used))
    k1, s_enc = 448 / A, 2688 / A
    n = near_code = near_scale = 0
    for r in range(rows):
        for b in range(cols // 16):
            blk = x[r, 16 * b:16 * b + 16].astype(np.float64)
            ab = Fraction(float(np.max(np.abs(blk))))
            si, sdist = rne_index(E4M3, ab * k1)
            got_s = int(q["scales"][r, b])
            if got_s != si:
                if strict:
                    assert sdist < TOL_SCALE, (r, b, got_s, si, float(sdist))
                else:
                    assert abs(got_s - si) == 1, (r, b, got_s, si)
                near_scale += 1
                continue
            dec = E4M3[si]
            for j in range(16):
                v = float(blk[j])
                neg = np.signbit(v)
                if dec == 0:
                    want, cdist = 0, Fraction(1)
                else:
                    want, cdist = rne_index(E2M1, abs(Fraction(v)) * s_enc / dec)
                got = nibble(q["codes"], r, 16 * b + j)
                assert (got >> 3) == int(neg), (r, b, j, v)
                if (got & 7) != want:
                    if strict:
                        assert cdist < TOL_CODE, (r, b, j, v, got & 7, want, float(cdist))
                    else:
                        assert abs((got & 7) - want) == 1, (r, b, j, v, got & 7, want)
                    near_code += 1
                n += 1
    return n, near_code, near_scale


def _rows(seed: int, rows: int, cols: int) -> np.ndarray:
    """Student-t(3) values with per-row magnitudes over six decades (block scales from E4M3's
    subnormal range to its top), 1% outliers x50, a few exact zeros and negative zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=(rows, cols)) * 10.0 ** rng.uniform(-6, 0, size=(rows, 1))
    out = rng.random((rows, cols)) < 0.01
    x[out] *= 50
    x = x.astype(np.float32)
    x[0, :16] = 0.0
    x[0, 16:20] = -0.0
    return x


@pytest.mark.parametrize("seed", [1, 2])
def test_1d_quantizer_matches_exact_definition(orc, seed):
    x = _rows(seed, 96, 256)
    q = orc.quantize_1d(x, RNE)
    n, near_code, near_scale = exact_block_check(x, q, q["amax"])
    assert n > 20000
    assert near_code + near_scale <= 3


def test_1d_quantizer_with_supplied_amax_matches_exact_definition(orc):
    x = _rows(3, 64, 128)
    A = float(np.max(np.abs(x))) * 3.7
    q = orc.quantize_1d(x, RNE, amax_in=A)
    n, near_code, near_scale = exact_block_check(x, q, A)
    assert n > 7000 and near_code + near_scale <= 3


def test_midpoint_values_round_to_even_exactly(orc):
    """Elements placed exactly on E2M1 midpoints of a block whose scale is exact: the oracle must
    land on the even code, as the exact definition does.  A = 2688 makes s_enc = 1 and k1 = 1/6;
    a block amax of 6 * 2^k gives the scale 2^k exactly, so z = x / 2^k with no rounding."""
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x = np.zeros((4, 16), dtype=np.float32)
    for r, k in enumerate([0, -2, 3, 5]):
        s = 2.0 ** k
        x[r, 0] = 6 * s                                       # the block amax
        x[r, 1:8] = [m * s for m in mids]
        x[r, 8:15] = [-m * s for m in mids]
    q = orc.quantize_1d(x, RNE, amax_in=2688.0)
    n, near_code, near_scale = exact_block_check(x, q, 2688.0)
    assert n == 64 and near_code == 0 and near_scale == 0


@pytest.mark.parametrize("seed", [0x51E40007, 12345])
def test_hadamard_transform_within_summation_bound_of_exact_product(orc, seed):
    rng = np.random.default_rng(seed % 997)
    T, F = 128, 48
    x = (rng.standard_t(3, size=(T, F)) * 10.0 ** rng.uniform(-3, 3, size=(1, F))).astype(np.float32)
    y = orc.hadamard_transform(x, seed).astype(np.float64)          # [F x T]
    H = scipy.linalg.hadamard(16).astype(np.float64)
    d = orc.rht_signs(seed).astype(np.float64)
    x64 = x.astype(np.float64)
    u = 2.0 ** -24
    for c in range(T // 16):
        chunk = x64[16 * c:16 * c + 16, :]                           # [16 x F]
        exact = (H @ (d[:, None] * chunk)) / 4                        # float64: exact here
        bound = 4 * u * np.sum(np.abs(chunk), axis=0) / 4             # 4 levels of fp32 adds
        err = np.abs(y[:, 16 * c:16 * c + 16].T - exact)
        assert np.all(err <= bound[None, :] * 1.0001), float(np.max(err / bound[None, :]))


def test_hadamard_quantize_matches_exact_quantization_of_exact_transform(orc):
    seed = 0x51E40009
    rng = np.random.default_rng(5)
    T, F = 64, 40
    x = (rng.standard_t(3, size=(T, F)) * 10.0 ** rng.uniform(-4, 0, size=(1, F))).astype(np.float32)
    q = orc.hadamard_quantize(x, seed, RNE)
    H = scipy.linalg.hadamard(16).astype(np.float64)
    d = orc.rht_signs(seed).astype(np.float64)
    yt = np.zeros((F, T))
    for c in range(T // 16):
        yt[:, 16 * c:16 * c + 16] = ((H @ (d[:, None] * x[16 * c:16 * c + 16, :].astype(np.float64))) / 4).T
    # the exact transform's amax and the oracle's fp32 one differ by at most its roundings
    assert abs(float(np.max(np.abs(yt))) - q["amax"]) <= 2 ** -21 * q["amax"]
    # against the exact transform the block step sees inputs off by the summation error, so
    # a few elements near a midpoint may land one code over; none may land further
    n, near_code, near_scale = exact_block_check(yt, q, q["amax"], strict=False)
    assert n >= F * T - 16 * near_scale and near_code + near_scale <= 0.002 * F * T
    # the oracle's own fp32 transform through the exact block step: midpoints only
    y32 = orc.hadamard_transform(x, seed)
    n, near_code, near_scale = exact_block_check(y32, q, q["amax"])
    assert n == F * T and near_code + near_scale <= 2
