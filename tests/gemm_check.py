"""The numeric bar for a GEMM output against the float64 oracle on the same quantized operands.

Two checks, both required:
- relative L2 (Frobenius) over the compared output <= 1e-5;
- every element within 1e-5 of the largest |reference| of its own output row, so that an error
  confined to a few elements cannot hide inside a norm.  (An all-zero reference row must then be
  matched exactly.)  The kernel's only rounding is fp32 accumulation of exact block products; the
  errors it leaves are around 1e-7 of a row's largest value, two orders inside this bound.
"""
import numpy as np

REL_L2 = 1e-5
ELEM_REL = 1e-5


def rel_l2(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_gemm_close(got, ref, what: str = "") -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if got.ndim == 1:
        got, ref = got[None, :], ref[None, :]
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = rel_l2(got, ref)
    assert err <= REL_L2, f"{what}: rel L2 {err:.3e}"
    row_max = np.abs(ref).max(axis=1, keepdims=True) if ref.size else ref
    diff = np.abs(got - ref)
    ok = diff <= ELEM_REL * row_max
    if not ok.all():
        r, c = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: element ({r}, {c}) off by {diff[r, c]:.3e}, row max "
                             f"{row_max[r, 0]:.3e} ({int((~ok).sum())} elements beyond 1e-5 of "
                             f"their row's max)")
    return err
