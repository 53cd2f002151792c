"""Pins for the oracle's quantizers: idempotence, grid membership, the max-code invariant, the
rounding error bound, 2D transpose invariance and the zero / signed-zero special cases."""
import numpy as np
import pytest
import torch

import workloads as W

E2M1_GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _e4m3(b):
    return torch.from_numpy(np.asarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _unpack(codes):
    lo = codes & 0xF
    hi = codes >> 4
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def _values(nibbles):
    mag = E2M1_GRID[nibbles & 7]
    return np.where(nibbles & 8, -mag, mag)


def _block_scale_per_element(q, rows, cols):
    s = _e4m3(q["scales"])
    if q["layout"] == 1:
        return np.repeat(np.repeat(s, 16, axis=0), 16, axis=1)
    return np.repeat(s, 16, axis=1)


INPUTS = {
    "fp32_outliers": lambda: W.small_fp32((64, 256), 101),
    "bf16_student_t": lambda: W.act((48, 512), 201),
    "bf16_weight": lambda: W.weight((64, 128), 202),
    "bf16_grad_spikes": lambda: W.grad((80, 256), 301),
}


@pytest.mark.parametrize("name", list(INPUTS))
def test_grid_membership_and_error_bound(orc, name):
    x = INPUTS[name]()
    xb = W.bits(x)
    rows, cols = x.shape
    q = orc.quantize_1d(xb)
    xf = x.to(torch.float64).numpy()
    assert q["amax"] == float(np.abs(xf).max())
    v = _values(_unpack(q["codes"]))
    s = _block_scale_per_element(q, rows, cols)
    xh = orc.dequantize(q, rows, cols).astype(np.float64)
    # dequantized value = v * scale * s_dec (the first product exact, one fp32 rounding)
    np.testing.assert_allclose(xh, v * s * q["s_dec"], rtol=2 ** -23, atol=0)
    # every element sits on the E2M1 grid times its block scale
    nz = s > 0
    ratio = xh[nz] / (s[nz] * np.float64(np.float32(q["s_dec"])))
    assert np.all(np.isin(np.round(np.abs(ratio), 6), E2M1_GRID))
    # rounding error bound: within half a grid step of the scaled input, or saturated at 6
    z = xf * (2688.0 / q["amax"]) / s.clip(min=1e-300) * nz
    step = np.where(np.abs(z) < 2, 0.5, np.where(np.abs(z) < 4, 1.0, 2.0))
    err = np.abs(np.abs(v) - np.minimum(np.abs(z), 6.0))
    assert np.all(err[nz] <= step[nz] / 2 * (1 + 1e-5) + 1e-6)
    # signs agree wherever the code is non-zero
    assert np.all(np.sign(v[v != 0]) == np.sign(xf[v != 0]))


@pytest.mark.parametrize("name", list(INPUTS))
def test_max_code_invariant(orc, name):
    x = INPUTS[name]()
    q = orc.quantize_1d(W.bits(x))
    v = np.abs(_values(_unpack(q["codes"]))).reshape(x.shape[0], -1, 16)
    s = q["scales"]
    normal = s >= 0x08                           # E4M3 exponent field >= 1
    assert np.all(v.max(axis=2)[normal] == 6.0)
    # the block holding the tensor amax gets the largest scale, 448
    xf = np.abs(x.to(torch.float64).numpy()).reshape(x.shape[0], -1, 16)
    r, b = np.unravel_index(np.argmax(xf.max(axis=2)), s.shape)
    assert s[r, b] == 0x7E


@pytest.mark.parametrize("name", list(INPUTS))
def test_idempotent_with_supplied_amax(orc, name):
    x = INPUTS[name]()
    rows, cols = x.shape
    q1 = orc.quantize_1d(W.bits(x))
    xh = orc.dequantize(q1, rows, cols)
    q2 = orc.quantize_1d(xh, amax_in=q1["amax"])
    if np.all(q1["scales"][q1["scales"] > 0] >= 0x08):
        np.testing.assert_array_equal(q2["codes"], q1["codes"])
        np.testing.assert_array_equal(q2["scales"], q1["scales"])
        assert q2["s_dec"] == q1["s_dec"]


def test_zero_and_signed_zero_blocks(orc):
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, :16] = -0.0
    x[1, 16:] = np.linspace(-1, 1, 16, dtype=np.float32)
    q = orc.quantize_1d(x)
    assert q["scales"][0, 0] == 0 and q["scales"][0, 1] == 0 and q["scales"][1, 0] == 0
    nib = _unpack(q["codes"])
    assert np.all(nib[0, :16] == 8) and np.all(nib[0, 16:] == 0)   # -0.0 keeps its sign
    assert q["scales"][1, 1] == 0x7E
    # an all-zero tensor: unit tensor scales, zero block scales, zero codes
    z = orc.quantize_1d(np.zeros((4, 64), dtype=np.float32))
    assert z["amax"] == 0.0 and z["s_dec"] == 1.0
    assert not z["scales"].any() and not z["codes"].any()


def test_2d_transpose_invariance(orc):
    w = W.weight((96, 160), 202)
    wb = W.bits(w)
    q = orc.quantize_2d(wb)
    qt = orc.quantize_2d(np.ascontiguousarray(wb.T))
    np.testing.assert_array_equal(q["codes_t"], qt["codes"])
    np.testing.assert_array_equal(q["scales_t"], qt["scales"])
    np.testing.assert_array_equal(qt["codes_t"], q["codes"])
    assert q["s_dec"] == qt["s_dec"]
    # transposed copy holds the same values at transposed positions
    np.testing.assert_array_equal(_unpack(q["codes_t"]), _unpack(q["codes"]).T)


def test_2d_tile_scale_is_tile_amax(orc):
    w = W.weight((64, 64), 5)
    q = orc.quantize_2d(W.bits(w))
    wf = np.abs(w.to(torch.float64).numpy())
    tiles = wf.reshape(4, 16, 4, 16).max(axis=(1, 3))
    k1 = np.float32(448.0) / np.float32(q["amax"])
    t = (tiles.astype(np.float32) * k1).astype(np.float32)
    ref = torch.from_numpy(np.minimum(t, np.float32(448))).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(q["scales"], ref)
    # 2D blocks with a normal scale contain a +-6 code
    v = np.abs(_values(_unpack(q["codes"]))).reshape(4, 16, 4, 16).max(axis=(1, 3))
    assert np.all(v[q["scales"] >= 8] == 6.0)


def test_shape_errors(orc):
    with pytest.raises(ValueError):
        orc.quantize_1d(np.zeros((4, 24), dtype=np.float32))
    with pytest.raises(ValueError):
        orc.quantize_2d(np.zeros((24, 32), dtype=np.float32))
    bad = np.zeros((2, 16), dtype=np.float32)
    bad[1, 3] = np.inf
    with pytest.raises(ValueError):
        orc.quantize_1d(bad)
