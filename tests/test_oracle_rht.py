"""Pins for the oracle's random Hadamard transform and the Hadamard-transpose quantizer."""
import numpy as np
import pytest
import scipy.linalg
import torch

import workloads as W


def test_transform_matrix_is_sylvester_hadamard(orc):
    ones = np.ones(16, dtype=np.int32)
    cols = [orc.rht16(np.eye(16, dtype=np.float32)[j], ones) * 4 for j in range(16)]
    H = np.stack(cols, axis=1).astype(np.float64)
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(16))
    np.testing.assert_array_equal(H @ H.T, 16 * np.eye(16))


@pytest.mark.parametrize("seed", [0, 1, 0x51E40004, 2 ** 63 + 5])
def test_signed_transform_equals_dense_product(orc, seed):
    d = orc.rht_signs(seed)
    assert set(np.unique(d)) <= {-1, 1}
    H = scipy.linalg.hadamard(16).astype(np.float64)
    rng = np.random.default_rng(seed % 1000)
    for _ in range(50):
        x = rng.integers(-512, 512, 16).astype(np.float32)       # small integers: exact in fp32
        y = orc.rht16(x, d)
        np.testing.assert_array_equal(y.astype(np.float64), H @ (d * x.astype(np.float64)) / 4)
        # (H D / 4) is orthogonal: D H / 4 undoes it
        back = d * (H @ y.astype(np.float64)) / 4
        np.testing.assert_array_equal(back, x.astype(np.float64))


def test_signs_depend_on_seed(orc):
    a, b = orc.rht_signs(1), orc.rht_signs(2)
    assert not np.array_equal(a, b)
    np.testing.assert_array_equal(orc.rht_signs(1), a)


def test_wgrad_product_is_preserved(orc):
    """(M dY)^T (M X) = dY^T X for M the block-diagonal (H D / 4) along tokens."""
    rng = np.random.default_rng(0)
    T, F1, F2 = 64, 5, 7
    dy = rng.standard_normal((T, F1))
    x = rng.standard_normal((T, F2))
    d = orc.rht_signs(99)
    H = scipy.linalg.hadamard(16) * d[None, :] / 4.0
    M = np.kron(np.eye(T // 16), H)
    np.testing.assert_allclose((M @ dy).T @ (M @ x), dy.T @ x, rtol=1e-12, atol=1e-12)


def _transform_exact(xf, d):
    """Dense float64 (H D / 4) on 16-token chunks; exact for the integer inputs used below."""
    T, F = xf.shape
    H = scipy.linalg.hadamard(16).astype(np.float64) * d[None, :] / 4.0
    return np.concatenate([H @ xf[c * 16:(c + 1) * 16] for c in range(T // 16)], axis=0)


@pytest.mark.parametrize("rounding", [0, 1])
def test_hadamard_quantize_is_transform_then_transposed_1d(orc, rounding):
    rng = np.random.default_rng(5)
    T, F = 64, 48
    xi = rng.integers(-256, 256, (T, F)).astype(np.float32)
    x = torch.from_numpy(xi).to(torch.bfloat16)                   # exact: |x| < 2^8
    seed, sign_seed = 0x5EED, 0x51E4
    q = orc.hadamard_quantize(W.bits(x), sign_seed, rounding=rounding, seed=seed)
    y = _transform_exact(xi.astype(np.float64), orc.rht_signs(sign_seed))
    yt = np.ascontiguousarray(y.T.astype(np.float32))              # [F x T], exact
    assert q["amax"] == float(np.abs(y).max()) == orc.hadamard_amax(W.bits(x), sign_seed)
    ref = orc.quantize_1d(yt, rounding=rounding, seed=seed)
    np.testing.assert_array_equal(q["codes"], ref["codes"])
    np.testing.assert_array_equal(q["scales"], ref["scales"])
    assert q["s_dec"] == ref["s_dec"]


def test_hadamard_transform_is_rht16_per_chunk_and_feeds_the_quantizer(orc):
    """The transposed transform equals rht16 applied to every 16-token chunk of every feature,
    its largest magnitude is the Hadamard amax, and its 1D quantization is the Hadamard
    quantizer's output."""
    x = W.grad((64, 24), 77)
    xb = W.bits(x)
    sign_seed = 0x51E4
    y = orc.hadamard_transform(xb, sign_seed)
    d = orc.rht_signs(sign_seed)
    xv = orc.values(xb).astype(np.float32)
    assert y.shape == (24, 64)
    for f in range(24):
        for c in range(4):
            np.testing.assert_array_equal(y[f, 16 * c:16 * c + 16], orc.rht16(xv[16 * c:16 * c + 16, f], d))
    assert float(np.abs(y).max()) == orc.hadamard_amax(xb, sign_seed)
    q = orc.hadamard_quantize(xb, sign_seed, rounding=1, seed=9)
    ref = orc.quantize_1d(y, rounding=1, seed=9)
    np.testing.assert_array_equal(q["codes"], ref["codes"])
    np.testing.assert_array_equal(q["scales"], ref["scales"])
