"""Pins for the oracle's random mappings and its per-tensor scales, checked against properties
that the pages and the mathematics fix rather than against the oracle's own formulas.

- Random Hadamard signs ("Entrenamiento de Modelos de Lenguaje con 4 Bits de Precision",
  Metodologia de Entrenamiento: random Hadamard transforms).  A random sign vector must have
  independent, balanced entries: over many sign seeds every entry is -1 half of the time and
  every pair of entries is uncorrelated.
- Stochastic-rounding draws ("FP4 All the Way", Describir: stochastic rounding in the backward
  and update passes).  Each element needs its own uniform draw: two elements never share one
  (the index -> draw map is injective) and draws of neighbouring elements, in the same Philox
  counter or the next one, are uncorrelated.
- Per-tensor scales ("I ricercatori di Nvidia ...", Come funziona NVFP4?: multi-level scaling).
  k1 = 448/A, s_enc = 2688/A and s_dec = A/2688 are each ONE correctly rounded fp32 division,
  checked against round-to-nearest-even of the exact rational quotient, computed here with
  integer arithmetic only.
"""
import math

import numpy as np
import pytest


# ---- random Hadamard signs ----------------------------------------------------------------------
def _sign_matrix(orc, seeds):
    return np.stack([orc.rht_signs(int(s)) for s in seeds]).astype(np.float64)


def test_hadamard_signs_balanced_and_pairwise_independent(orc):
    n = 20000
    seeds = np.random.default_rng(0x5A17).integers(0, 2 ** 63, n, dtype=np.int64).astype(np.uint64)
    D = _sign_matrix(orc, seeds)                          # [n, 16] of +-1
    assert set(np.unique(D)) == {-1.0, 1.0}
    tol = 5.0 / math.sqrt(n)                              # 5 sigma of a mean of n +-1 variables
    freq_neg = (D < 0).mean(axis=0)                       # P(d_j = -1) = 1/2
    assert np.all(np.abs(freq_neg - 0.5) <= 0.5 * tol), freq_neg
    prod = (D.T @ D) / n                                  # E[d_i d_j] = 0 for i != j
    iu = np.triu_indices(16, 1)
    assert len(iu[0]) == 120
    assert np.all(np.abs(prod[iu]) <= tol), np.abs(prod[iu]).max()


def test_hadamard_signs_consecutive_seeds_independent(orc):
    """Seeds 0, 1, 2, ... (a caller's per-layer counter) still give unrelated sign vectors."""
    n = 20000
    D = _sign_matrix(orc, np.arange(n, dtype=np.uint64))
    tol = 5.0 / math.sqrt(n)
    assert np.all(np.abs((D < 0).mean(axis=0) - 0.5) <= 0.5 * tol)
    # entry j of seed s against entry j of seed s + 1: uncorrelated
    lag = (D[1:] * D[:-1]).mean(axis=0)
    assert np.all(np.abs(lag) <= 5.0 / math.sqrt(n - 1)), lag
    # all 2^16 vectors are possible; 20000 draws of a uniform 16-bit vector repeat ~3000 times
    # at most by the birthday bound (expected 2900); a mapping using fewer bits repeats far more
    keys = ((D < 0).astype(np.int64) * (1 << np.arange(16))).sum(axis=1)
    dup = n - len(np.unique(keys))
    assert dup < 3600, dup


# ---- stochastic-rounding draws ------------------------------------------------------------------
def test_sr_draws_injective_over_index_range(orc):
    """Distinct element indices never share a draw: the 48-bit fingerprint (r16 under three
    seeds) of every index is unique.  A chance collision of two distinct draws under all three
    seeds has probability 2^-48 per pair (~0.004 expected over the ~1.4e12 pairs here)."""
    lo = np.arange(1 << 20, dtype=np.uint64)
    hi = (np.uint64(1) << np.uint64(35)) + np.arange(1 << 16, dtype=np.uint64)   # counter high word
    top = (np.uint64(1) << np.uint64(62)) + np.arange(1 << 12, dtype=np.uint64)
    idx = np.concatenate([lo, hi, top])
    fp = np.zeros(idx.shape, dtype=np.uint64)
    for s in (0x5EED0003, 7, 2 ** 63 + 11):
        fp = (fp << np.uint64(16)) | orc.sr_bits_n(s, idx).astype(np.uint64)
    assert np.all(orc.sr_bits_n(3, idx) < 65536)
    assert len(np.unique(fp)) == len(idx)


def test_sr_draws_uncorrelated_within_and_across_counters(orc):
    """At p = 1/2 the round-up event is r16 < 2^15.  Over 10^5 seeds, the 16 elements of two
    adjacent Philox counters (indices 8c .. 8c + 15) round up independently: each with
    frequency 1/2 and every one of the 120 pairs uncorrelated, within 5 sigma.  The same holds
    for the raw 16-bit values (uniform mean 1/2, pairwise correlation 0)."""
    n = 100000
    rng = np.random.default_rng(0xC0FFEE)
    seeds = rng.integers(0, 2 ** 63, n, dtype=np.int64).astype(np.uint64)
    base = np.uint64(8 * 12345)
    idx = base + np.arange(16, dtype=np.uint64)
    R = np.stack([orc.sr_bits_n(int(s), idx) for s in seeds]).astype(np.float64)   # [n, 16]
    tol = 5.0 / math.sqrt(n)
    up = (R < 32768).astype(np.float64)
    assert np.all(np.abs(up.mean(axis=0) - 0.5) <= 0.5 * tol)
    iu = np.triu_indices(16, 1)
    c_up = np.corrcoef(up, rowvar=False)[iu]
    assert np.all(np.abs(c_up) <= tol), np.abs(c_up).max()
    u = (R + 0.5) / 65536.0
    assert np.all(np.abs(u.mean(axis=0) - 0.5) <= tol * math.sqrt(1 / 12))
    c_u = np.corrcoef(u, rowvar=False)[iu]
    assert np.all(np.abs(c_u) <= tol), np.abs(c_u).max()


def test_sr_round_up_rate_is_p_for_every_element_slot(orc):
    """For each of the eight slots sharing a counter, the round-up frequency of an element with
    p = (|z| - lo)/(hi - lo) = 0.3 is 0.3 (within 5 sigma over 4*10^4 counters)."""
    n = 40000
    idx = np.arange(8 * n, dtype=np.uint64)
    r = orc.sr_bits_n(0x5EED0004, idx).reshape(n, 8)
    z = np.float32(0.5 + 0.3 * 0.5)                          # lo = 0.5, hi = 1.0, p = 0.3
    codes = orc.e2m1_sr_n(np.full(r.shape, z, np.float32), r.astype(np.uint32))
    up = (codes == 2).mean(axis=0)
    assert set(np.unique(codes)) <= {1, 2}
    sig = math.sqrt(0.3 * 0.7 / n)
    assert np.all(np.abs(up - 0.3) <= 5 * sig), up


# ---- per-tensor scales: one correctly rounded division each -------------------------------------
def _f32_parts(a: np.float32):
    """(m, e) with a = m * 2^e exactly, m an integer (a > 0, finite)."""
    bits = int(np.asarray(a, np.float32).view(np.uint32))
    ex, fr = (bits >> 23) & 0xFF, bits & 0x7FFFFF
    if ex == 0:
        return fr, -149
    return fr | 0x800000, ex - 150


def _rne_f32_of_ratio(num: int, num_e: int, den: int, den_e: int) -> np.float32:
    """Round-to-nearest-even to binary32 of (num * 2^num_e) / (den * 2^den_e), num, den > 0
    integers, using integer arithmetic only (normals and subnormals; no overflow expected)."""
    # exponent of the quotient's leading bit: 2^L <= q < 2^(L+1)
    L = (num.bit_length() - den.bit_length()) + (num_e - den_e)
    n2, d2 = num, den
    sh = num_e - den_e
    if sh >= 0:
        n2 <<= sh
    else:
        d2 <<= -sh
    # now q = n2 / d2 exactly; fix L so that 2^L <= q < 2^(L+1)
    def ge(L):                       # q >= 2^L ?
        return (n2 << max(-L, 0)) >= (d2 << max(L, 0))
    while not ge(L):
        L -= 1
    while ge(L + 1):
        L += 1
    e = max(L - 23, -149)            # exponent of the last kept bit (subnormals: fixed at -149)
    if e >= 0:
        qi, r = divmod(n2, d2 << e)
        den_r = d2 << e
    else:
        qi, r = divmod(n2 << -e, d2)
        den_r = d2
    if 2 * r > den_r or (2 * r == den_r and (qi & 1)):
        qi += 1
    return np.float32(math.ldexp(qi, e))


def _random_amaxes(n, seed):
    rng = np.random.default_rng(seed)
    lo = int(np.float32(2.0 ** -100).view(np.uint32))
    hi = int(np.finfo(np.float32).max.view(np.uint32))
    bits = rng.integers(lo, hi + 1, n, dtype=np.int64).astype(np.uint32)
    special = np.array([2.0 ** -100, 3.0, 448.0, 2688.0, 1.0, 6.0, 7.0, 10.5, 1e-30, 1e30,
                        np.finfo(np.float32).max, np.float32(np.float32(2.0 ** -100) * np.float32(1.0000001))],
                       dtype=np.float32)
    return np.concatenate([bits.view(np.float32), special])


def test_rne_ratio_helper_against_known_values():
    """The integer rounding used as the reference is itself checked on exact and tie cases."""
    assert _rne_f32_of_ratio(448, 0, 3, 0) == np.float32(149.33333)
    assert _rne_f32_of_ratio(1, 0, 3, 0) == np.float32(1.0) / np.float32(3.0)
    # 1 + 2^-24 is a tie between 1 and 1 + 2^-23: even is 1
    assert _rne_f32_of_ratio((1 << 24) + 1, -24, 1, 0) == np.float32(1.0)
    # 1 + 3 * 2^-24 ties between 1 + 2^-23 and 1 + 2^-22: even is 1 + 2^-22
    assert _rne_f32_of_ratio((1 << 24) + 3, -24, 1, 0) == np.float32(1.0 + 2.0 ** -22)
    # subnormal: 2^-149 * 1.5 ties to 2 * 2^-149
    assert _rne_f32_of_ratio(3, -150, 1, 0) == np.float32(2.0 ** -148)
    # numpy's float64 -> float32 rounding agrees where the quotient is exact in float64
    rng = np.random.default_rng(4)
    for a, b in rng.integers(1, 1 << 20, (2000, 2)):
        if (int(a) << 40) % int(b) == 0:
            continue
        q = _rne_f32_of_ratio(int(a), 0, int(b), 0)
        assert q == np.float32(np.float32(a) / np.float32(b))


def test_tensor_scales_are_single_correctly_rounded_divisions(orc):
    A = _random_amaxes(100000, 0x7E45)
    for a in A:
        k1, s_enc, s_dec = orc.tensor_scales(a)
        m, e = _f32_parts(a)
        assert np.float32(k1) == _rne_f32_of_ratio(448, 0, m, e), (a, k1)
        assert np.float32(s_enc) == _rne_f32_of_ratio(2688, 0, m, e), (a, s_enc)
        assert np.float32(s_dec) == _rne_f32_of_ratio(m, e, 2688, 0), (a, s_dec)


def test_tensor_scales_zero_threshold(orc):
    """Below 2^-100 (zero included) the tensor counts as all-zero: k1 = 448, s_enc = s_dec = 1."""
    t = np.float32(2.0 ** -100)
    for a in (0.0, np.nextafter(t, np.float32(0)), np.float32(1e-40), np.float32(2.0 ** -120)):
        assert orc.tensor_scales(a) == (448.0, 1.0, 1.0)
    k1, s_enc, s_dec = orc.tensor_scales(t)
    assert (k1, s_enc, s_dec) != (448.0, 1.0, 1.0)
    assert np.float32(s_dec) == _rne_f32_of_ratio(1, -100, 2688, 0)
