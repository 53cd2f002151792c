"""CPU oracle for the NVFP4 hot path (ctypes wrapper over ``nvfp4_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import this package.  The product library (``nvfp4_bit_quantized_amd``)
never imports, links or calls it, and the two share no code: the oracle is plain C compiled with
gcc, the product is HIP compiled for gfx950.

Arrays are numpy.  bf16 tensors are passed as their raw ``uint16`` bit patterns; fp32 as
``float32``.  Every function mirrors one function of ``nvfp4_oracle.c``, whose comments cite the
passage of the pages each step follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra"]

F32, BF16 = 0, 1
RNE, SR = 0, 1
L1x16, L16x16 = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = C.CDLL(_LIB_PATH)
        P = C.c_void_p
        i64, u64, i32, f32 = C.c_int64, C.c_uint64, C.c_int, C.c_float
        L.or_e2m1_value.restype = C.c_double
        L.or_e2m1_value.argtypes = [C.c_uint]
        L.or_e2m1_rne.restype = C.c_uint
        L.or_e2m1_rne.argtypes = [f32]
        L.or_e2m1_sr.restype = C.c_uint
        L.or_e2m1_sr.argtypes = [f32, C.c_uint]
        L.or_e4m3_value.restype = C.c_double
        L.or_e4m3_value.argtypes = [C.c_uint]
        L.or_e4m3_rne_sat.restype = C.c_uint
        L.or_e4m3_rne_sat.argtypes = [f32]
        L.or_philox4x32_10.restype = None
        L.or_philox4x32_10.argtypes = [P, P, P]
        L.or_sr_bits.restype = C.c_uint
        L.or_sr_bits.argtypes = [u64, u64]
        L.or_f32_to_bf16.restype = C.c_uint16
        L.or_f32_to_bf16.argtypes = [f32]
        L.or_tensor_scales.restype = None
        L.or_tensor_scales.argtypes = [f32, P]
        L.or_amax.restype = i32
        L.or_amax.argtypes = [P, i32, i64, i64, i64, P]
        L.or_quantize_1d.restype = i32
        L.or_quantize_1d.argtypes = [P, i32, i64, i64, i64, P, i32, u64, P, P, P, P]
        L.or_quantize_2d.restype = i32
        L.or_quantize_2d.argtypes = [P, i32, i64, i64, i64, P, P, P, P, P, P, P]
        L.or_rht_signs.restype = None
        L.or_rht_signs.argtypes = [u64, P]
        L.or_rht16.restype = None
        L.or_rht16.argtypes = [P, P]
        L.or_hadamard_amax.restype = i32
        L.or_hadamard_amax.argtypes = [P, i32, i64, i64, i64, u64, P]
        L.or_hadamard_transform.restype = i32
        L.or_hadamard_transform.argtypes = [P, i32, i64, i64, i64, u64, P]
        L.or_hadamard_quantize.restype = i32
        L.or_hadamard_quantize.argtypes = [P, i32, i64, i64, i64, u64, P, i32, u64, P, P, P, P]
        L.or_dequantize.restype = i32
        L.or_dequantize.argtypes = [P, P, i32, f32, i64, i64, i32, P, i64]
        L.or_gemm_f64.restype = i32
        L.or_gemm_f64.argtypes = [P, P, i32, f32, P, P, i32, f32, i64, i64, i64, P, i64, P]
        L.or_mx_quantize_1d.restype = i32
        L.or_mx_quantize_1d.argtypes = [P, i32, i64, i64, i64, i32, u64, P, P]
        L.or_mx_dequantize.restype = i32
        L.or_mx_dequantize.argtypes = [P, P, i64, i64, P, i64]
        L.or_mx_gemm_f64.restype = i32
        L.or_mx_gemm_f64.argtypes = [P, P, P, P, i64, i64, i64, P, i64, P]
        L.or_qdq.restype = i32
        L.or_qdq.argtypes = [P, i32, i64, i64, i64, i32, i32, P, i32, u64, P, P]
        L.or_e2m1_rne_n.restype = None
        L.or_e2m1_rne_n.argtypes = [P, i64, P]
        L.or_e2m1_sr_n.restype = None
        L.or_e2m1_sr_n.argtypes = [P, P, i64, P]
        L.or_e4m3_rne_sat_n.restype = None
        L.or_e4m3_rne_sat_n.argtypes = [P, i64, P]
        L.or_sr_bits_n.restype = None
        L.or_sr_bits_n.argtypes = [u64, P, i64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return a.ctypes.data


def _input(x: np.ndarray):
    """(contiguous array, dtype code) for a float32 array or raw bf16 uint16 bits."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle input must be float32 or bf16 bits (uint16), got {x.dtype}")


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ---- scalar codecs -------------------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return lib().or_e2m1_value(int(code))


def e2m1_rne(z: float) -> int:
    return lib().or_e2m1_rne(float(z))


def e2m1_sr(z: float, r16: int) -> int:
    return lib().or_e2m1_sr(float(z), int(r16))


def e4m3_value(b: int) -> float:
    return lib().or_e4m3_value(int(b))


def e4m3_rne_sat(t: float) -> int:
    return lib().or_e4m3_rne_sat(float(t))


def f32_to_bf16(f: float) -> int:
    return lib().or_f32_to_bf16(float(f))


def e2m1_rne_n(z: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32)
    out = np.zeros(z.shape, dtype=np.uint8)
    lib().or_e2m1_rne_n(_ptr(z), z.size, _ptr(out))
    return out


def e2m1_sr_n(z: np.ndarray, r16: np.ndarray) -> np.ndarray:
    z = np.ascontiguousarray(z, dtype=np.float32)
    r = np.ascontiguousarray(np.broadcast_to(r16, z.shape), dtype=np.uint32)
    out = np.zeros(z.shape, dtype=np.uint8)
    lib().or_e2m1_sr_n(_ptr(z), _ptr(r), z.size, _ptr(out))
    return out


def e4m3_rne_sat_n(t: np.ndarray) -> np.ndarray:
    t = np.ascontiguousarray(t, dtype=np.float32)
    out = np.zeros(t.shape, dtype=np.uint8)
    lib().or_e4m3_rne_sat_n(_ptr(t), t.size, _ptr(out))
    return out


def sr_bits_n(seed: int, idx: np.ndarray) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.uint64)
    out = np.zeros(idx.shape, dtype=np.uint32)
    lib().or_sr_bits_n(int(seed), _ptr(idx), idx.size, _ptr(out))
    return out


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.asarray(ctr, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().or_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_bits(seed: int, idx: int) -> int:
    return lib().or_sr_bits(int(seed), int(idx))


def tensor_scales(A: float):
    out = np.zeros(3, dtype=np.float32)
    lib().or_tensor_scales(float(A), _ptr(out))
    return float(out[0]), float(out[1]), float(out[2])


# ---- tensor operations ---------------------------------------------------------------------------
def amax(x: np.ndarray) -> float:
    x, dt = _input(x)
    rows, cols = x.shape
    out = np.zeros(1, dtype=np.float32)
    _check(lib().or_amax(_ptr(x), dt, rows, cols, cols, _ptr(out)), "amax")
    return float(out[0])


def quantize_1d(x: np.ndarray, rounding: int = RNE, seed: int = 0, amax_in: float | None = None):
    """Returns dict(codes [R x K/2] u8, scales [R x K/16] u8, amax, s_dec)."""
    x, dt = _input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    am = np.zeros(1, dtype=np.float32)
    sd = np.zeros(1, dtype=np.float32)
    ain = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    _check(lib().or_quantize_1d(_ptr(x), dt, rows, cols, cols, _ptr(ain), int(rounding), int(seed),
                                _ptr(codes), _ptr(scales), _ptr(am), _ptr(sd)), "quantize_1d")
    return dict(codes=codes, scales=scales, amax=float(am[0]), s_dec=float(sd[0]), layout=L1x16)


def quantize_2d(w: np.ndarray, amax_in: float | None = None, transposed: bool = True):
    """Returns dict(codes, scales [R/16 x K/16], codes_t [K x R/2], scales_t, amax, s_dec)."""
    w, dt = _input(w)
    rows, cols = w.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows // 16, cols // 16), dtype=np.uint8)
    codes_t = np.zeros((cols, rows // 2), dtype=np.uint8) if transposed else None
    scales_t = np.zeros((cols // 16, rows // 16), dtype=np.uint8) if transposed else None
    am = np.zeros(1, dtype=np.float32)
    sd = np.zeros(1, dtype=np.float32)
    ain = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    _check(lib().or_quantize_2d(_ptr(w), dt, rows, cols, cols, _ptr(ain), _ptr(codes), _ptr(scales),
                                _ptr(codes_t), _ptr(scales_t), _ptr(am), _ptr(sd)), "quantize_2d")
    return dict(codes=codes, scales=scales, codes_t=codes_t, scales_t=scales_t,
                amax=float(am[0]), s_dec=float(sd[0]), layout=L16x16)


def rht_signs(sign_seed: int) -> np.ndarray:
    d = np.zeros(16, dtype=np.int32)
    lib().or_rht_signs(int(sign_seed), _ptr(d))
    return d


def rht16(x: np.ndarray, d: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    dd = np.ascontiguousarray(d, dtype=np.int32)
    assert y.shape == (16,) and dd.shape == (16,)
    lib().or_rht16(_ptr(y), _ptr(dd))
    return y


def hadamard_amax(x: np.ndarray, sign_seed: int) -> float:
    x, dt = _input(x)
    T, F = x.shape
    out = np.zeros(1, dtype=np.float32)
    _check(lib().or_hadamard_amax(_ptr(x), dt, T, F, F, int(sign_seed), _ptr(out)), "hadamard_amax")
    return float(out[0])


def hadamard_transform(x: np.ndarray, sign_seed: int) -> np.ndarray:
    """x [T x F] -> the transformed, transposed tensor y [F x T] float32 that
    ``hadamard_quantize`` encodes: y[f, 16c:16c+16] = rht16(x[16c:16c+16, f])."""
    x, dt = _input(x)
    T, F = x.shape
    y = np.zeros((F, T), dtype=np.float32)
    _check(lib().or_hadamard_transform(_ptr(x), dt, T, F, F, int(sign_seed), _ptr(y)),
           "hadamard_transform")
    return y


def hadamard_quantize(x: np.ndarray, sign_seed: int, rounding: int = RNE, seed: int = 0,
                      amax_in: float | None = None):
    """x [T x F] -> dict(codes [F x T/2], scales [F x T/16], amax, s_dec)."""
    x, dt = _input(x)
    T, F = x.shape
    codes = np.zeros((F, T // 2), dtype=np.uint8)
    scales = np.zeros((F, T // 16), dtype=np.uint8)
    am = np.zeros(1, dtype=np.float32)
    sd = np.zeros(1, dtype=np.float32)
    ain = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    _check(lib().or_hadamard_quantize(_ptr(x), dt, T, F, F, int(sign_seed), _ptr(ain), int(rounding),
                                      int(seed), _ptr(codes), _ptr(scales), _ptr(am), _ptr(sd)),
           "hadamard_quantize")
    return dict(codes=codes, scales=scales, amax=float(am[0]), s_dec=float(sd[0]), layout=L1x16)


def dequantize(q: dict, rows: int, cols: int, out_bf16: bool = False) -> np.ndarray:
    codes = np.ascontiguousarray(q["codes"])
    scales = np.ascontiguousarray(q["scales"])
    out = np.zeros((rows, cols), dtype=np.uint16 if out_bf16 else np.float32)
    _check(lib().or_dequantize(_ptr(codes), _ptr(scales), int(q["layout"]), float(q["s_dec"]),
                               rows, cols, BF16 if out_bf16 else F32, _ptr(out), cols), "dequantize")
    return out


def values(x: np.ndarray) -> np.ndarray:
    """float64 values of a float32 array or of raw bf16 bits (the upper half of an fp32)."""
    x, dt = _input(x)
    if dt == BF16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def quant_noise(x: np.ndarray, q: dict) -> tuple[float, float]:
    """Quantization-noise diagnostic ("FP4 All the Way", Describir: quantized training loses
    efficiency once the gradient norm falls below about sqrt(3) times the quantization noise):
    (sum x^2, sum (Q(x) - x)^2) in float64, with Q(x) the dequantized tensor (``dequantize``)."""
    xv = values(x)
    rows, cols = xv.shape
    qv = dequantize(q, rows, cols).astype(np.float64)
    return float(np.sum(xv * xv)), float(np.sum((qv - xv) ** 2))


def qdq(x: np.ndarray, block: int, scale_fmt: int, rounding: int = RNE, seed: int = 0,
        amax_in: float | None = None):
    """Format sweep: quantize with `block` elements per scale (8, 16, 32) and scale format
    `scale_fmt` (0: E4M3 under the fp32 tensor scale; 1: E8M0 power of two), dequantize.
    Returns (y float32 [rows x cols], tensor amax used (0 for E8M0))."""
    x, dt = _input(x)
    rows, cols = x.shape
    y = np.zeros((rows, cols), dtype=np.float32)
    am = np.zeros(1, dtype=np.float32)
    ain = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    _check(lib().or_qdq(_ptr(x), dt, rows, cols, cols, int(block), int(scale_fmt), _ptr(ain),
                        int(rounding), int(seed), _ptr(y), _ptr(am)), "qdq")
    return y, float(am[0])


def gemm_f64(a: dict, b: dict, M: int, N: int, K: int, rows: np.ndarray | None = None) -> np.ndarray:
    """C = A * B^T in float64 for the selected rows of A (all rows if None)."""
    rsel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rsel is None else len(rsel)
    out = np.zeros((nrows, N), dtype=np.float64)
    ac, asc = np.ascontiguousarray(a["codes"]), np.ascontiguousarray(a["scales"])
    bc, bsc = np.ascontiguousarray(b["codes"]), np.ascontiguousarray(b["scales"])
    _check(lib().or_gemm_f64(_ptr(ac), _ptr(asc), int(a["layout"]), float(a["s_dec"]),
                             _ptr(bc), _ptr(bsc), int(b["layout"]), float(b["s_dec"]),
                             M, N, K, _ptr(rsel), nrows, _ptr(out)), "gemm_f64")
    return out


def mx_quantize_1d(x: np.ndarray, rounding: int = RNE, seed: int = 0):
    x, dt = _input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    _check(lib().or_mx_quantize_1d(_ptr(x), dt, rows, cols, cols, int(rounding), int(seed),
                                   _ptr(codes), _ptr(scales)), "mx_quantize_1d")
    return dict(codes=codes, scales=scales)


def mx_dequantize(q: dict, rows: int, cols: int) -> np.ndarray:
    out = np.zeros((rows, cols), dtype=np.float32)
    _check(lib().or_mx_dequantize(_ptr(np.ascontiguousarray(q["codes"])),
                                  _ptr(np.ascontiguousarray(q["scales"])), rows, cols, _ptr(out), cols),
           "mx_dequantize")
    return out


def mx_gemm_f64(a: dict, b: dict, M: int, N: int, K: int, rows: np.ndarray | None = None) -> np.ndarray:
    rsel = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nrows = M if rsel is None else len(rsel)
    out = np.zeros((nrows, N), dtype=np.float64)
    _check(lib().or_mx_gemm_f64(_ptr(np.ascontiguousarray(a["codes"])), _ptr(np.ascontiguousarray(a["scales"])),
                                _ptr(np.ascontiguousarray(b["codes"])), _ptr(np.ascontiguousarray(b["scales"])),
                                M, N, K, _ptr(rsel), nrows, _ptr(out)), "mx_gemm_f64")
    return out
