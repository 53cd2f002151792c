"""Pins for the oracle GEMM (NVFP4 and MXFP4): exact rational brute force on tiny shapes, a
closed form, agreement with a library matmul of the dequantized operands, and MXFP4 scale rules."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_mags():
    with open(os.path.join(GOLDEN, "e2m1_value_set.txt")) as f:
        return [Fraction(l.strip()) for l in f if l.strip() and not l.startswith("#")]


def _e4m3_frac(b):
    v = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).item()
    return Fraction(v)


def _nib(codes, r, k):
    b = int(codes[r, k // 2])
    return (b >> 4) if k & 1 else (b & 0xF)


def _frac_val(c, mags):
    v = mags[c & 7]
    return -v if c & 8 else v


def _random_q(rng, rows, K, layout):
    codes = rng.integers(0, 256, (rows, K // 2), dtype=np.uint8)
    srows = rows // 16 if layout == 1 else rows
    scales = rng.integers(0, 0x7F, (srows, K // 16), dtype=np.uint8)
    return dict(codes=codes, scales=scales, layout=layout,
                s_dec=float(np.float32(rng.uniform(1e-4, 1e-2))))


@pytest.mark.parametrize("M,N,K,lb", [(8, 8, 16, 0), (16, 32, 32, 1), (32, 16, 64, 0), (5, 16, 48, 1)])
def test_gemm_matches_exact_rational_sum(orc, M, N, K, lb):
    rng = np.random.default_rng(M * 1000 + N + K)
    mags = _page_mags()
    a = _random_q(rng, M, K, 0)
    b = _random_q(rng, N, K, lb)
    got = orc.gemm_f64(a, b, M, N, K)
    sdec = Fraction(a["s_dec"]) * Fraction(b["s_dec"])
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                sa = _e4m3_frac(int(a["scales"][m, k // 16]))
                sb = _e4m3_frac(int(b["scales"][(n // 16) if lb else n, k // 16]))
                acc += _frac_val(_nib(a["codes"], m, k), mags) * sa * \
                       _frac_val(_nib(b["codes"], n, k), mags) * sb
            exact = acc * sdec
            if exact == 0:
                assert got[m, n] == 0
            else:
                assert abs(Fraction(got[m, n]) - exact) <= abs(exact) * Fraction(1, 10 ** 15) + \
                    Fraction(1, 10 ** 300)


def test_gemm_closed_form_all_ones(orc):
    M, N, K = 16, 32, 256
    ones = lambda r: dict(codes=np.full((r, K // 2), 0x22, np.uint8),     # 1.0 | 1.0 << 4
                          scales=np.full((r, K // 16), 0x38, np.uint8),    # E4M3 1.0
                          layout=0, s_dec=0.5)
    got = orc.gemm_f64(ones(M), ones(N), M, N, K)
    np.testing.assert_array_equal(got, np.full((M, N), K * 0.25))


def test_gemm_matches_library_matmul_of_dequantized(orc):
    x = W.act((64, 256), 11)
    w = W.weight((48, 256), 12)
    qa = orc.quantize_1d(W.bits(x))
    qb = orc.quantize_2d(W.bits(w))
    c = orc.gemm_f64(qa, qb, 64, 48, 256)
    # dequantized operands (each element v*s exact, times s_dec rounded once in fp32) give the
    # same product up to that one rounding per element
    da = orc.dequantize(qa, 64, 256).astype(np.float64)
    db = orc.dequantize(qb, 48, 256).astype(np.float64)
    ref = torch.from_numpy(da) @ torch.from_numpy(db).T
    rel = np.linalg.norm(c - ref.numpy()) / np.linalg.norm(ref.numpy())
    assert rel < 1e-6
    # and the quantized product is close to the bf16 product (a 4-bit sanity bound)
    full = x.double() @ w.double().T
    assert np.linalg.norm(c - full.numpy()) / np.linalg.norm(full.numpy()) < 0.25


def test_gemm_row_selection(orc):
    rng = np.random.default_rng(1)
    a = _random_q(rng, 40, 64, 0)
    b = _random_q(rng, 24, 64, 0)
    full = orc.gemm_f64(a, b, 40, 24, 64)
    rows = np.array([39, 0, 17, 17])
    np.testing.assert_array_equal(orc.gemm_f64(a, b, 40, 24, 64, rows=rows), full[rows])


# ---- MXFP4 --------------------------------------------------------------------------------------
def test_mx_scale_rule(orc):
    x = np.zeros((4, 64), dtype=np.float32)
    x[0, :32] = 1.0                 # floor(log2 1) - 2 = -2 -> byte 125, codes 4.0
    x[1, :32] = 6.0                 # floor(log2 6) - 2 = 0 -> byte 127, codes 6.0
    x[2, 5] = 0.75                  # floor(log2 .75) - 2 = -3 -> 0.75 * 8 = 6
    x[3, 32:] = np.float32(2.0 ** -130)   # subnormal block: clamped exponent -127
    q = orc.mx_quantize_1d(x)
    assert q["scales"][0, 0] == 125 and q["scales"][0, 1] == 127      # zero block -> 2^0
    assert np.all(q["codes"][0, :16] == 0x66)
    assert q["scales"][1, 0] == 127 and np.all(q["codes"][1, :16] == 0x77)
    assert q["scales"][2, 0] == 124
    assert (q["codes"][2, 2] >> 4) == 7
    assert q["scales"][3, 1] == 0
    d = orc.mx_dequantize(q, 4, 64)
    np.testing.assert_array_equal(d[0, :32], 1.0)
    np.testing.assert_array_equal(d[1, :32], 6.0)


def test_mx_power_of_two_scaling_is_exact(orc):
    x = W.act((32, 128), 3)
    q = orc.mx_quantize_1d(W.bits(x))
    xf = x.float().numpy()
    e = q["scales"].astype(np.int64) - 127
    z = xf * np.exp2(-np.repeat(e, 32, axis=1)).astype(np.float64)
    assert np.all(np.abs(z) < 8)
    # codes are the RNE of the exactly scaled values
    np.testing.assert_array_equal(
        orc.e2m1_rne_n(z.astype(np.float32)).reshape(32, 64, 2),
        np.stack([q["codes"] & 0xF, q["codes"] >> 4], axis=-1))


def test_mx_gemm_matches_exact_rational_sum(orc):
    rng = np.random.default_rng(9)
    mags = _page_mags()
    M, N, K = 6, 5, 64
    a = dict(codes=rng.integers(0, 256, (M, K // 2), dtype=np.uint8),
             scales=rng.integers(110, 140, (M, K // 32), dtype=np.uint8))
    b = dict(codes=rng.integers(0, 256, (N, K // 2), dtype=np.uint8),
             scales=rng.integers(110, 140, (N, K // 32), dtype=np.uint8))
    got = orc.mx_gemm_f64(a, b, M, N, K)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                e = int(a["scales"][m, k // 32]) + int(b["scales"][n, k // 32]) - 254
                acc += _frac_val(_nib(a["codes"], m, k), mags) * \
                       _frac_val(_nib(b["codes"], n, k), mags) * Fraction(2) ** e
            assert Fraction(got[m, n]) == acc
