"""Python binding of ``libnvfp4.so`` (the NVFP4 hot path on MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared in
``include/nvfp4.h``.  PyTorch provides device memory and the current HIP stream.  There is no
fallback: if the library is missing or the GPU is absent, calls raise.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_LAYOUT, ERR_LAUNCH, ERR_SCRATCH = range(8)
F32, BF16 = 0, 1
RNE, SR = 0, 1
BLK_1x16, BLK_16x16, MX_1x32 = 0, 1, 2

SYMBOLS = ("nvfp4_status_string", "nvfp4_amax", "nvfp4_hadamard_amax", "nvfp4_quantize_1d",
           "nvfp4_quantize_2d", "nvfp4_hadamard_quantize", "nvfp4_dequantize", "nvfp4_gemm",
           "mxfp4_quantize_1d", "mxfp4_gemm", "nvfp4_dual_amax", "nvfp4_quantize_dual",
           "nvfp4_quantize_1d_noise", "nvfp4_qdq", "mxfp4_quantize_1d_t", "nvfp4_amax_accumulate",
           "nvfp4_hadamard_amax_accumulate", "nvfp4_hadamard_quantize_noise", "nvfp4_gemm_ws",
           "nvfp4_gemm_workspace_size", "nvfp4_gemm_ws_noalloc", "mxfp4_gemm_ws",
           "mxfp4_gemm_workspace_size", "mxfp4_quantize_dual", "nvfp4_dual_amax_accumulate")


class NvTensor(C.Structure):
    """Mirror of ``nvfp4_tensor``."""
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("amax", C.c_void_p),
                ("s_dec", C.c_void_p), ("rows", C.c_int64), ("cols", C.c_int64),
                ("layout", C.c_int32), ("reserved", C.c_int32)]


_lib = None


def lib():
    """Load ``libnvfp4.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        P, i64, u64, i32 = C.c_void_p, C.c_int64, C.c_uint64, C.c_int
        T = C.POINTER(NvTensor)
        L.nvfp4_status_string.restype = C.c_char_p
        L.nvfp4_status_string.argtypes = [i32]
        L.nvfp4_amax.argtypes = [P, i32, i64, i64, i64, P, P]
        L.nvfp4_hadamard_amax.argtypes = [P, i32, i64, i64, i64, u64, P, P]
        L.nvfp4_amax_accumulate.argtypes = [P, i32, i64, i64, i64, P, P]
        L.nvfp4_hadamard_amax_accumulate.argtypes = [P, i32, i64, i64, i64, u64, P, P]
        L.nvfp4_quantize_1d.argtypes = [P, i32, i64, P, i32, u64, T, P]
        L.nvfp4_quantize_2d.argtypes = [P, i32, i64, P, T, T, P]
        L.nvfp4_hadamard_quantize.argtypes = [P, i32, i64, u64, P, i32, u64, T, P]
        L.nvfp4_hadamard_quantize_noise.argtypes = [P, i32, i64, u64, P, i32, u64, T, P, P]
        L.nvfp4_dequantize.argtypes = [T, P, i32, i64, P]
        L.nvfp4_gemm.argtypes = [T, T, P, i32, i64, P]
        L.nvfp4_gemm_ws.argtypes = [T, T, P, i32, i64, P, C.c_size_t, P]
        L.nvfp4_gemm_workspace_size.argtypes = [i64, i64, i64, C.POINTER(C.c_size_t)]
        L.nvfp4_gemm_ws_noalloc.argtypes = [T, T, P, i32, i64, P]
        L.mxfp4_gemm_ws.argtypes = [T, T, P, i32, i64, P, C.c_size_t, P]
        L.mxfp4_gemm_workspace_size.argtypes = [i64, i64, i64, C.POINTER(C.c_size_t)]
        L.mxfp4_quantize_1d.argtypes = [P, i32, i64, i32, u64, T, P]
        L.mxfp4_gemm.argtypes = [T, T, P, i32, i64, P]
        L.mxfp4_quantize_1d_t.argtypes = [P, i32, i64, i32, u64, T, P]
        L.mxfp4_quantize_dual.argtypes = [P, i32, i64, i32, u64, u64, T, T, P]
        L.nvfp4_dual_amax.argtypes = [P, i32, i64, i64, i64, u64, P, P, P]
        L.nvfp4_dual_amax_accumulate.argtypes = [P, i32, i64, i64, i64, u64, P, P, P]
        L.nvfp4_quantize_dual.argtypes = [P, i32, i64, u64, P, P, i32, u64, u64, T, T, P]
        L.nvfp4_quantize_1d_noise.argtypes = [P, i32, i64, P, i32, u64, T, P, P]
        L.nvfp4_qdq.argtypes = [P, i32, i64, i64, i64, i32, i32, P, i32, u64, P, i64, P, P, P]
        for name in SYMBOLS[1:]:
            getattr(L, name).restype = i32
        _lib = L
    return _lib


class Nvfp4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().nvfp4_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def _check(fn: str, status: int):
    if status != OK:
        raise Nvfp4Error(fn, status)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")


def _ptr(t: torch.Tensor | None) -> int | None:
    """Device address of a GPU tensor; a host tensor is refused here, since a kernel handed a host
    address would fault instead of returning an error."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    return t.data_ptr()


@dataclass
class QTensor:
    """An NVFP4 (or MXFP4) matrix in device memory: logical [rows x cols], cols contiguous."""
    codes: torch.Tensor          # uint8 [rows, cols/2]
    scales: torch.Tensor         # uint8, shape per layout
    amax: torch.Tensor | None    # float32 [1]
    s_dec: torch.Tensor | None   # float32 [1]
    rows: int
    cols: int
    layout: int

    def desc(self) -> NvTensor:
        return NvTensor(_ptr(self.codes), _ptr(self.scales), _ptr(self.amax), _ptr(self.s_dec),
                        self.rows, self.cols, self.layout, 0)

    @staticmethod
    def empty(rows: int, cols: int, layout: int = BLK_1x16, device="cuda") -> "QTensor":
        u8 = dict(dtype=torch.uint8, device=device)
        if layout == BLK_16x16:
            scales = torch.empty((rows // 16, cols // 16), **u8)
        elif layout == MX_1x32:
            scales = torch.empty((rows, cols // 32), **u8)
        else:
            scales = torch.empty((rows, cols // 16), **u8)
        f = dict(dtype=torch.float32, device=device)
        nv = layout != MX_1x32
        return QTensor(torch.empty((rows, cols // 2), **u8), scales,
                       torch.empty(1, **f) if nv else None, torch.empty(1, **f) if nv else None,
                       rows, cols, layout)


def _x(x: torch.Tensor):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with unit column stride")
    return x, _dtype_code(x.dtype), x.stride(0)


def amax(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    x, dt, ld = _x(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    _check("nvfp4_amax", lib().nvfp4_amax(_ptr(x), dt, x.shape[0], x.shape[1], ld, _ptr(out),
                                          _stream(x.device)))
    return out


def hadamard_amax(x: torch.Tensor, sign_seed: int, out: torch.Tensor | None = None) -> torch.Tensor:
    x, dt, ld = _x(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    _check("nvfp4_hadamard_amax", lib().nvfp4_hadamard_amax(_ptr(x), dt, x.shape[0], x.shape[1], ld,
                                                            sign_seed, _ptr(out), _stream(x.device)))
    return out


def amax_accumulate(x: torch.Tensor, acc: torch.Tensor) -> torch.Tensor:
    """acc (device fp32 [1], caller-initialised, >= 0) <- max(acc, max |x|); no zero-fill."""
    x, dt, ld = _x(x)
    _check("nvfp4_amax_accumulate", lib().nvfp4_amax_accumulate(_ptr(x), dt, x.shape[0], x.shape[1],
                                                                ld, _ptr(acc), _stream(x.device)))
    return acc


def hadamard_amax_accumulate(x: torch.Tensor, sign_seed: int, acc: torch.Tensor) -> torch.Tensor:
    """acc <- max(acc, amax of the random Hadamard transform of x); no zero-fill."""
    x, dt, ld = _x(x)
    _check("nvfp4_hadamard_amax_accumulate",
           lib().nvfp4_hadamard_amax_accumulate(_ptr(x), dt, x.shape[0], x.shape[1], ld, sign_seed,
                                                _ptr(acc), _stream(x.device)))
    return acc


def quantize_1d(x: torch.Tensor, rounding: int = RNE, seed: int = 0,
                amax_in: torch.Tensor | None = None, out: QTensor | None = None) -> QTensor:
    x, dt, ld = _x(x)
    q = QTensor.empty(x.shape[0], x.shape[1], BLK_1x16, x.device) if out is None else out
    d = q.desc()
    _check("nvfp4_quantize_1d", lib().nvfp4_quantize_1d(_ptr(x), dt, ld, _ptr(amax_in), rounding,
                                                        seed, C.byref(d), _stream(x.device)))
    return q


def quantize_1d_noise(x: torch.Tensor, rounding: int = SR, seed: int = 0,
                      amax_in: torch.Tensor | None = None, out: QTensor | None = None,
                      sums: torch.Tensor | None = None):
    """quantize_1d plus the noise diagnostic: (QTensor, sums) with sums a device float64 [2] =
    (sum x^2, sum (Q(x) - x)^2).  ``diagnostics.noise_report(sums)`` reads them on the host."""
    x, dt, ld = _x(x)
    q = QTensor.empty(x.shape[0], x.shape[1], BLK_1x16, x.device) if out is None else out
    sums = torch.empty(2, dtype=torch.float64, device=x.device) if sums is None else sums
    d = q.desc()
    _check("nvfp4_quantize_1d_noise",
           lib().nvfp4_quantize_1d_noise(_ptr(x), dt, ld, _ptr(amax_in), rounding, seed,
                                         C.byref(d), _ptr(sums), _stream(x.device)))
    return q, sums


E4M3, E8M0 = 0, 1


def qdq(x: torch.Tensor, block: int, scale_fmt: int, rounding: int = RNE, seed: int = 0,
        amax_in: torch.Tensor | None = None, out: torch.Tensor | None = None,
        sums: torch.Tensor | None = None, amax_out: torch.Tensor | None = None):
    """Format sweep: x quantized with `block` (8/16/32) elements per scale in `scale_fmt` (E4M3
    under the tensor scale, or E8M0) and dequantized -> (y fp32, amax used, sums)."""
    x, dt, ld = _x(x)
    y = torch.empty(x.shape, dtype=torch.float32, device=x.device) if out is None else out
    amax_out = torch.empty(1, dtype=torch.float32, device=x.device) if amax_out is None else amax_out
    _check("nvfp4_qdq", lib().nvfp4_qdq(_ptr(x), dt, x.shape[0], x.shape[1], ld, block, scale_fmt,
                                        _ptr(amax_in), rounding, seed, _ptr(y), y.stride(0),
                                        _ptr(amax_out), _ptr(sums), _stream(x.device)))
    return y, amax_out, sums


def quantize_2d(w: torch.Tensor, transposed: bool = True, amax_in: torch.Tensor | None = None,
                out: QTensor | None = None, out_t: QTensor | None = None):
    """Returns (Q, Q^T) -- Q^T is None unless ``transposed``."""
    w, dt, ld = _x(w)
    q = QTensor.empty(w.shape[0], w.shape[1], BLK_16x16, w.device) if out is None else out
    qt = None
    if transposed:
        qt = QTensor.empty(w.shape[1], w.shape[0], BLK_16x16, w.device) if out_t is None else out_t
    d = q.desc()
    dt_ = qt.desc() if qt is not None else None
    _check("nvfp4_quantize_2d", lib().nvfp4_quantize_2d(_ptr(w), dt, ld, _ptr(amax_in), C.byref(d),
                                                        C.byref(dt_) if dt_ is not None else None,
                                                        _stream(w.device)))
    return q, qt


def hadamard_quantize(x: torch.Tensor, sign_seed: int, rounding: int = RNE, seed: int = 0,
                      amax_in: torch.Tensor | None = None, out: QTensor | None = None) -> QTensor:
    """x [T tokens x F features] -> NVFP4 [F x T] of the random-Hadamard-transformed tensor."""
    x, dt, ld = _x(x)
    T, F = x.shape
    q = QTensor.empty(F, T, BLK_1x16, x.device) if out is None else out
    d = q.desc()
    _check("nvfp4_hadamard_quantize",
           lib().nvfp4_hadamard_quantize(_ptr(x), dt, ld, sign_seed, _ptr(amax_in), rounding, seed,
                                         C.byref(d), _stream(x.device)))
    return q


def hadamard_quantize_noise(x: torch.Tensor, sign_seed: int, rounding: int = SR, seed: int = 0,
                            amax_in: torch.Tensor | None = None, out: QTensor | None = None,
                            sums: torch.Tensor | None = None):
    """hadamard_quantize plus the noise diagnostic of the transformed tensor y it encodes:
    (QTensor [F x T], sums) with sums a device float64 [2] = (sum y^2, sum (Q(y) - y)^2)."""
    x, dt, ld = _x(x)
    T, F = x.shape
    q = QTensor.empty(F, T, BLK_1x16, x.device) if out is None else out
    sums = torch.empty(2, dtype=torch.float64, device=x.device) if sums is None else sums
    d = q.desc()
    _check("nvfp4_hadamard_quantize_noise",
           lib().nvfp4_hadamard_quantize_noise(_ptr(x), dt, ld, sign_seed, _ptr(amax_in), rounding,
                                               seed, C.byref(d), _ptr(sums), _stream(x.device)))
    return q, sums


def dual_amax(x: torch.Tensor, sign_seed: int, out: torch.Tensor | None = None,
              out_t: torch.Tensor | None = None):
    """(amax of x, amax of its random Hadamard transform) from one read of x [T x F]."""
    x, dt, ld = _x(x)
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    out_t = torch.empty(1, dtype=torch.float32, device=x.device) if out_t is None else out_t
    _check("nvfp4_dual_amax", lib().nvfp4_dual_amax(_ptr(x), dt, x.shape[0], x.shape[1], ld,
                                                    sign_seed, _ptr(out), _ptr(out_t),
                                                    _stream(x.device)))
    return out, out_t


def dual_amax_accumulate(x: torch.Tensor, sign_seed: int, acc: torch.Tensor, acc_t: torch.Tensor):
    """acc <- max(acc, amax of x), acc_t <- max(acc_t, amax of its random Hadamard transform),
    from one read of x [T x F]; both caller-initialised (>= 0), no zero-fill."""
    x, dt, ld = _x(x)
    _check("nvfp4_dual_amax_accumulate",
           lib().nvfp4_dual_amax_accumulate(_ptr(x), dt, x.shape[0], x.shape[1], ld, sign_seed,
                                            _ptr(acc), _ptr(acc_t), _stream(x.device)))
    return acc, acc_t


def quantize_dual(x: torch.Tensor, sign_seed: int, rounding: int = RNE, seed: int = 0,
                  seed_t: int = 0, amax_in: torch.Tensor | None = None,
                  amax_t_in: torch.Tensor | None = None, out: QTensor | None = None,
                  out_t: QTensor | None = None):
    """x [T x F] -> (row-wise NVFP4 [T x F], Hadamard-transformed NVFP4 [F x T]) from one read."""
    x, dt, ld = _x(x)
    T, F = x.shape
    q = QTensor.empty(T, F, BLK_1x16, x.device) if out is None else out
    qt = QTensor.empty(F, T, BLK_1x16, x.device) if out_t is None else out_t
    d, dt_ = q.desc(), qt.desc()
    _check("nvfp4_quantize_dual",
           lib().nvfp4_quantize_dual(_ptr(x), dt, ld, sign_seed, _ptr(amax_in), _ptr(amax_t_in),
                                     rounding, seed, seed_t, C.byref(d), C.byref(dt_),
                                     _stream(x.device)))
    return q, qt


def dequantize(q: QTensor, dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None):
    y = torch.empty((q.rows, q.cols), dtype=dtype, device=q.codes.device) if out is None else out
    d = q.desc()
    _check("nvfp4_dequantize", lib().nvfp4_dequantize(C.byref(d), _ptr(y), _dtype_code(y.dtype),
                                                      y.stride(0), _stream(y.device)))
    return y


def gemm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace with which ``nvfp4_gemm_ws`` splits an M x N x K GEMM (0: no split)."""
    n = C.c_size_t(0)
    _check("nvfp4_gemm_workspace_size", lib().nvfp4_gemm_workspace_size(M, N, K, C.byref(n)))
    return int(n.value)


def gemm(a: QTensor, b: QTensor, dtype: torch.dtype = torch.float32,
         out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
         split: bool = True) -> torch.Tensor:
    """C = A * B^T (A [M x K], B [N x K]) with fp32 accumulation.  With ``split`` (the default)
    the call is ``nvfp4_gemm_ws``: a partly empty last round of output tiles is split along K into
    the workspace (``workspace``, a uint8 device tensor, or one allocated here when it is needed);
    ``split=False`` calls ``nvfp4_gemm``."""
    c = torch.empty((a.rows, b.rows), dtype=dtype, device=a.codes.device) if out is None else out
    da, db = a.desc(), b.desc()
    if not split:
        _check("nvfp4_gemm", lib().nvfp4_gemm(C.byref(da), C.byref(db), _ptr(c),
                                              _dtype_code(c.dtype), c.stride(0), _stream(c.device)))
        return c
    need = gemm_workspace_size(a.rows, b.rows, a.cols)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=c.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("nvfp4_gemm_ws", lib().nvfp4_gemm_ws(C.byref(da), C.byref(db), _ptr(c),
                                                _dtype_code(c.dtype), c.stride(0), _ptr(workspace),
                                                nbytes, _stream(c.device)))
    return c


def mx_quantize_1d(x: torch.Tensor, rounding: int = RNE, seed: int = 0,
                   out: QTensor | None = None) -> QTensor:
    x, dt, ld = _x(x)
    q = QTensor.empty(x.shape[0], x.shape[1], MX_1x32, x.device) if out is None else out
    d = q.desc()
    _check("mxfp4_quantize_1d", lib().mxfp4_quantize_1d(_ptr(x), dt, ld, rounding, seed, C.byref(d),
                                                        _stream(x.device)))
    return q


def mx_quantize_1d_t(x: torch.Tensor, rounding: int = RNE, seed: int = 0,
                     out: QTensor | None = None) -> QTensor:
    """x [T x F] -> MXFP4 of x^T [F x T] (32-token blocks), read once."""
    x, dt, ld = _x(x)
    q = QTensor.empty(x.shape[1], x.shape[0], MX_1x32, x.device) if out is None else out
    d = q.desc()
    _check("mxfp4_quantize_1d_t", lib().mxfp4_quantize_1d_t(_ptr(x), dt, ld, rounding, seed,
                                                            C.byref(d), _stream(x.device)))
    return q


def mx_quantize_dual(x: torch.Tensor, rounding: int = RNE, seed: int = 0, seed_t: int = 0,
                     out: QTensor | None = None, out_t: QTensor | None = None):
    """x [T x F] -> (row-wise MXFP4 [T x F], MXFP4 of x^T [F x T]) from one read."""
    x, dt, ld = _x(x)
    T, F = x.shape
    q = QTensor.empty(T, F, MX_1x32, x.device) if out is None else out
    qt = QTensor.empty(F, T, MX_1x32, x.device) if out_t is None else out_t
    d, dt_ = q.desc(), qt.desc()
    _check("mxfp4_quantize_dual",
           lib().mxfp4_quantize_dual(_ptr(x), dt, ld, rounding, seed, seed_t, C.byref(d),
                                     C.byref(dt_), _stream(x.device)))
    return q, qt


def mx_gemm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace with which ``mxfp4_gemm_ws`` splits an M x N x K GEMM (0: no split)."""
    n = C.c_size_t(0)
    _check("mxfp4_gemm_workspace_size", lib().mxfp4_gemm_workspace_size(M, N, K, C.byref(n)))
    return int(n.value)


def mx_gemm(a: QTensor, b: QTensor, dtype: torch.dtype = torch.float32,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
            split: bool = True) -> torch.Tensor:
    """C = A * B^T for MXFP4 operands; ``split`` and ``workspace`` as for ``gemm``."""
    c = torch.empty((a.rows, b.rows), dtype=dtype, device=a.codes.device) if out is None else out
    da, db = a.desc(), b.desc()
    if not split:
        _check("mxfp4_gemm", lib().mxfp4_gemm(C.byref(da), C.byref(db), _ptr(c),
                                              _dtype_code(c.dtype), c.stride(0), _stream(c.device)))
        return c
    need = mx_gemm_workspace_size(a.rows, b.rows, a.cols)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=c.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("mxfp4_gemm_ws", lib().mxfp4_gemm_ws(C.byref(da), C.byref(db), _ptr(c),
                                                _dtype_code(c.dtype), c.stride(0), _ptr(workspace),
                                                nbytes, _stream(c.device)))
    return c
