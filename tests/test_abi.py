"""C-ABI contract checks that run without a GPU: the library loads, exports every function that
include/nvfp4.h declares, and rejects bad arguments before anything is enqueued (only argument
combinations that fail validation are passed, so no kernel is ever launched here)."""
import ctypes as C
import os
import re

import pytest

import nvfp4_bit_quantized_amd as nv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:nvfp4|mxfp4)_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nv.LIB_PATH):
        pytest.skip("libnvfp4.so not built")
    return nv.lib()


def test_exports_every_declared_function(L):
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(nv.SYMBOLS)


def test_exports_nothing_else(L):
    """The dynamic symbol table holds exactly the declared functions (kernel handles and helpers
    are local), read from the ELF file with the system's nm."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", nv.LIB_PATH], check=True,
                         capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    syms -= {"_init", "_fini"}
    assert syms == set(_declared()), sorted(syms ^ set(_declared()))


def test_status_strings(L):
    for s in range(8):
        assert L.nvfp4_status_string(s)
    assert L.nvfp4_status_string(99) == b"unknown status"


FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below fails validation


def _q(rows, cols, layout=nv.BLK_1x16, codes=FAKE, scales=FAKE, amax=FAKE, sdec=FAKE, reserved=0):
    return nv.NvTensor(codes, scales, amax, sdec, rows, cols, layout, reserved)


def test_quantize_validation(L):
    q = _q(8, 32)
    assert L.nvfp4_quantize_1d(None, nv.BF16, 32, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_NULL
    assert L.nvfp4_quantize_1d(FAKE, 7, 32, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_DTYPE
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, 5, 0, C.byref(q), None) == nv.ERR_DTYPE
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 16, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_SHAPE
    assert L.nvfp4_quantize_1d(FAKE + 2, nv.BF16, 32, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_ALIGN
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 36, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_ALIGN
    bad = _q(8, 24)
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, nv.RNE, 0, C.byref(bad), None) == nv.ERR_SHAPE
    wrong = _q(8, 32, layout=nv.BLK_16x16)
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, nv.RNE, 0, C.byref(wrong), None) == nv.ERR_LAYOUT
    noamax = _q(8, 32, amax=None)
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, nv.RNE, 0, C.byref(noamax), None) == nv.ERR_NULL
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, nv.RNE, 0, None, None) == nv.ERR_NULL
    res = _q(8, 32, reserved=1)
    assert L.nvfp4_quantize_1d(FAKE, nv.BF16, 32, None, nv.RNE, 0, C.byref(res), None) == nv.ERR_LAYOUT


def test_quantize_2d_and_hadamard_validation(L):
    w = _q(24, 32, layout=nv.BLK_16x16)          # rows not a multiple of 16
    assert L.nvfp4_quantize_2d(FAKE, nv.BF16, 32, None, C.byref(w), None, None) == nv.ERR_SHAPE
    w = _q(32, 48, layout=nv.BLK_16x16)
    wt = _q(32, 48, layout=nv.BLK_16x16)         # transposed copy must be [48 x 32]
    assert L.nvfp4_quantize_2d(FAKE, nv.BF16, 48, None, C.byref(w), C.byref(wt), None) == nv.ERR_SHAPE
    h = _q(12, 40)                               # F=12 features (not a multiple of 8), T=40 (not %16)
    assert L.nvfp4_hadamard_quantize(FAKE, nv.BF16, 16, 1, None, nv.RNE, 0, C.byref(h), None) == nv.ERR_SHAPE
    assert L.nvfp4_hadamard_amax(FAKE, nv.BF16, 40, 16, 16, 1, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_hadamard_amax(FAKE, nv.BF16, 32, 16, 16, 1, None, None) == nv.ERR_NULL
    assert L.nvfp4_amax(FAKE, nv.BF16, 4, 16, 16, FAKE + 1, None) == nv.ERR_ALIGN


def test_documented_multiple_of_8_rules(L):
    """nvfp4_amax needs cols % 8 == 0 and every Hadamard call F % 8 == 0 (with T % 16 == 0 met),
    as include/nvfp4.h states; each violation alone gives NVFP4_ERR_SHAPE."""
    for cols in (4, 12, 20):
        assert L.nvfp4_amax(FAKE, nv.BF16, 4, cols, 32, FAKE, None) == nv.ERR_SHAPE
        assert L.nvfp4_amax_accumulate(FAKE, nv.BF16, 4, cols, 32, FAKE, None) == nv.ERR_SHAPE
    for F in (4, 12, 20):
        assert L.nvfp4_hadamard_amax(FAKE, nv.BF16, 32, F, 32, 1, FAKE, None) == nv.ERR_SHAPE
        assert L.nvfp4_hadamard_amax_accumulate(FAKE, nv.BF16, 32, F, 32, 1, FAKE, None) == nv.ERR_SHAPE
        q = _q(F, 32)                            # out [F x T=32]: T is fine, F is not
        assert L.nvfp4_hadamard_quantize(FAKE, nv.BF16, 32, 1, None, nv.RNE, 0, C.byref(q), None) == nv.ERR_SHAPE
        assert L.nvfp4_hadamard_quantize_noise(FAKE, nv.BF16, 32, 1, None, nv.SR, 0, C.byref(q), FAKE,
                                               None) == nv.ERR_SHAPE


def test_amax_accumulate_validation(L):
    """The accumulating amax calls validate like the plain ones (nothing is enqueued)."""
    assert L.nvfp4_amax_accumulate(None, nv.BF16, 4, 16, 16, FAKE, None) == nv.ERR_NULL
    assert L.nvfp4_amax_accumulate(FAKE, nv.BF16, 4, 16, 16, None, None) == nv.ERR_NULL
    assert L.nvfp4_amax_accumulate(FAKE, nv.BF16, 4, 16, 16, FAKE + 1, None) == nv.ERR_ALIGN
    assert L.nvfp4_amax_accumulate(FAKE, nv.BF16, 4, 12, 16, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_amax_accumulate(FAKE, 7, 4, 16, 16, FAKE, None) == nv.ERR_DTYPE
    assert L.nvfp4_hadamard_amax_accumulate(FAKE, nv.BF16, 40, 16, 16, 1, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_hadamard_amax_accumulate(FAKE, nv.BF16, 32, 12, 16, 1, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_hadamard_amax_accumulate(FAKE, nv.BF16, 32, 16, 16, 1, None, None) == nv.ERR_NULL
    assert L.nvfp4_hadamard_amax_accumulate(FAKE, nv.BF16, 32, 16, 16, 1, FAKE + 2, None) == nv.ERR_ALIGN


def test_hadamard_noise_validation(L):
    q = _q(16, 32)                               # out [F=16 x T=32]
    assert L.nvfp4_hadamard_quantize_noise(FAKE, nv.BF16, 16, 1, None, nv.SR, 0, C.byref(q), None,
                                           None) == nv.ERR_NULL
    assert L.nvfp4_hadamard_quantize_noise(FAKE, nv.BF16, 16, 1, None, nv.SR, 0, C.byref(q),
                                           FAKE + 4, None) == nv.ERR_ALIGN
    bad = _q(12, 32)                             # F = 12 features: not a multiple of 8
    assert L.nvfp4_hadamard_quantize_noise(FAKE, nv.BF16, 16, 1, None, nv.SR, 0, C.byref(bad),
                                           FAKE, None) == nv.ERR_SHAPE


def test_gemm_validation(L):
    a, b = _q(64, 64), _q(32, 48)
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), FAKE, nv.F32, 32, None) == nv.ERR_SHAPE
    b = _q(32, 64, layout=nv.MX_1x32)
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), FAKE, nv.F32, 32, None) == nv.ERR_LAYOUT
    b = _q(32, 64)
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), FAKE, nv.F32, 16, None) == nv.ERR_SHAPE
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), None, nv.F32, 32, None) == nv.ERR_NULL
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), FAKE, 9, 32, None) == nv.ERR_DTYPE
    nos = _q(32, 64, sdec=None)
    assert L.nvfp4_gemm(C.byref(a), C.byref(nos), FAKE, nv.F32, 32, None) == nv.ERR_NULL
    mxa, mxb = _q(64, 48, layout=nv.MX_1x32), _q(32, 48, layout=nv.MX_1x32)
    assert L.mxfp4_gemm(C.byref(mxa), C.byref(mxb), FAKE, nv.F32, 32, None) == nv.ERR_SHAPE
    assert L.mxfp4_quantize_1d(FAKE, nv.BF16, 48, nv.RNE, 0, C.byref(mxa), None) == nv.ERR_SHAPE


def test_mx_transposed_validation(L):
    # out [F x T] = [64 x 96]: x is [96 x 64]
    q = _q(64, 96, layout=nv.MX_1x32)
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 64, 2, 0, C.byref(q), None) == nv.ERR_DTYPE
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 32, nv.RNE, 0, C.byref(q), None) == nv.ERR_SHAPE
    assert L.mxfp4_quantize_1d_t(None, nv.BF16, 64, nv.RNE, 0, C.byref(q), None) == nv.ERR_NULL
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 64, nv.RNE, 0, None, None) == nv.ERR_NULL
    odd = _q(60, 96, layout=nv.MX_1x32)                      # F % 8 != 0
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 64, nv.RNE, 0, C.byref(odd), None) == nv.ERR_SHAPE
    short = _q(64, 32 * 3 + 16, layout=nv.MX_1x32)            # T % 32 != 0 fails the layout check
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 64, nv.RNE, 0, C.byref(short), None) == nv.ERR_SHAPE
    nv_layout = _q(64, 96)
    assert L.mxfp4_quantize_1d_t(FAKE, nv.BF16, 64, nv.RNE, 0, C.byref(nv_layout), None) == nv.ERR_LAYOUT


def test_mx_dual_validation(L):
    # x [T x F] = [96 x 64]: out [96 x 64], out_t [64 x 96]
    q, qt = _q(96, 64, layout=nv.MX_1x32), _q(64, 96, layout=nv.MX_1x32)
    f = L.mxfp4_quantize_dual
    assert f(FAKE, nv.BF16, 64, 2, 0, 0, C.byref(q), C.byref(qt), None) == nv.ERR_DTYPE
    assert f(FAKE, nv.BF16, 32, nv.RNE, 0, 0, C.byref(q), C.byref(qt), None) == nv.ERR_SHAPE
    assert f(None, nv.BF16, 64, nv.RNE, 0, 0, C.byref(q), C.byref(qt), None) == nv.ERR_NULL
    assert f(FAKE, nv.BF16, 64, nv.RNE, 0, 0, None, C.byref(qt), None) == nv.ERR_NULL
    assert f(FAKE, nv.BF16, 64, nv.RNE, 0, 0, C.byref(q), None, None) == nv.ERR_NULL
    wrong_t = _q(64, 64, layout=nv.MX_1x32)                  # not [F x T]
    assert f(FAKE, nv.BF16, 64, nv.RNE, 0, 0, C.byref(q), C.byref(wrong_t), None) == nv.ERR_SHAPE
    q48, qt48 = _q(48, 64, layout=nv.MX_1x32), _q(64, 48, layout=nv.MX_1x32)   # T % 32 != 0
    assert f(FAKE, nv.BF16, 64, nv.RNE, 0, 0, C.byref(q48), C.byref(qt48), None) == nv.ERR_SHAPE
    f48, ft48 = _q(96, 48, layout=nv.MX_1x32), _q(48, 96, layout=nv.MX_1x32)   # F % 32 != 0
    assert f(FAKE, nv.BF16, 48, nv.RNE, 0, 0, C.byref(f48), C.byref(ft48), None) == nv.ERR_SHAPE
    nv_layout = _q(96, 64)
    assert f(FAKE, nv.BF16, 64, nv.RNE, 0, 0, C.byref(nv_layout), C.byref(qt), None) == nv.ERR_LAYOUT

def test_dual_amax_accumulate_validation(L):
    f = L.nvfp4_dual_amax_accumulate
    assert f(FAKE, nv.BF16, 24, 64, 64, 0, FAKE, FAKE + 4, None) == nv.ERR_SHAPE       # T % 16
    assert f(FAKE, nv.BF16, 32, 60, 64, 0, FAKE, FAKE + 4, None) == nv.ERR_SHAPE       # F % 8
    assert f(FAKE, nv.BF16, 32, 64, 64, 0, None, FAKE + 4, None) == nv.ERR_NULL
    assert f(FAKE, nv.BF16, 32, 64, 64, 0, FAKE, None, None) == nv.ERR_NULL
    assert f(FAKE, nv.BF16, 32, 64, 64, 0, FAKE + 2, FAKE + 4, None) == nv.ERR_ALIGN
    assert f(FAKE, nv.BF16, 32, 64, 64, 0, FAKE, FAKE, None) == nv.ERR_SHAPE           # same slot
    assert f(None, nv.BF16, 32, 64, 64, 0, FAKE, FAKE + 4, None) == nv.ERR_NULL

def test_dequantize_validation(L):
    q = _q(16, 32)
    assert L.nvfp4_dequantize(C.byref(q), None, nv.F32, 32, None) == nv.ERR_NULL
    assert L.nvfp4_dequantize(C.byref(q), FAKE, nv.F32, 8, None) == nv.ERR_SHAPE
    assert L.nvfp4_dequantize(None, FAKE, nv.F32, 32, None) == nv.ERR_NULL
    bad = _q(16, 32, layout=7)
    assert L.nvfp4_dequantize(C.byref(bad), FAKE, nv.F32, 32, None) == nv.ERR_LAYOUT


def test_dual_validation(L):
    assert L.nvfp4_dual_amax(FAKE, nv.BF16, 40, 16, 16, 1, FAKE, FAKE + 4, None) == nv.ERR_SHAPE
    assert L.nvfp4_dual_amax(FAKE, nv.BF16, 32, 16, 16, 1, None, FAKE, None) == nv.ERR_NULL
    assert L.nvfp4_dual_amax(FAKE, nv.BF16, 32, 16, 16, 1, FAKE, FAKE, None) == nv.ERR_SHAPE
    assert L.nvfp4_dual_amax(FAKE, nv.BF16, 32, 16, 16, 1, FAKE, FAKE + 2, None) == nv.ERR_ALIGN
    q, qt = _q(32, 48), _q(48, 32, amax=FAKE + 4, sdec=FAKE + 8)
    assert L.nvfp4_quantize_dual(FAKE, nv.BF16, 48, 1, None, None, nv.RNE, 0, 0, C.byref(q),
                                 None, None) == nv.ERR_NULL
    assert L.nvfp4_quantize_dual(FAKE, nv.BF16, 48, 1, None, None, 5, 0, 0, C.byref(q),
                                 C.byref(qt), None) == nv.ERR_DTYPE
    wrong = _q(32, 32, amax=FAKE + 4, sdec=FAKE + 8)
    assert L.nvfp4_quantize_dual(FAKE, nv.BF16, 48, 1, None, None, nv.RNE, 0, 0, C.byref(q),
                                 C.byref(wrong), None) == nv.ERR_SHAPE
    same = _q(48, 32)
    assert L.nvfp4_quantize_dual(FAKE, nv.BF16, 48, 1, None, None, nv.RNE, 0, 0, C.byref(q),
                                 C.byref(same), None) == nv.ERR_SHAPE
    mx = _q(48, 32, layout=nv.MX_1x32, amax=FAKE + 4, sdec=FAKE + 8)
    assert L.nvfp4_quantize_dual(FAKE, nv.BF16, 48, 1, None, None, nv.RNE, 0, 0, C.byref(q),
                                 C.byref(mx), None) == nv.ERR_LAYOUT
    assert L.nvfp4_quantize_dual(FAKE + 2, nv.BF16, 48, 1, None, None, nv.RNE, 0, 0, C.byref(q),
                                 C.byref(qt), None) == nv.ERR_ALIGN


def test_noise_validation(L):
    q = _q(8, 32)
    assert L.nvfp4_quantize_1d_noise(FAKE, nv.BF16, 32, None, nv.SR, 0, C.byref(q), None,
                                     None) == nv.ERR_NULL
    assert L.nvfp4_quantize_1d_noise(FAKE, nv.BF16, 32, None, nv.SR, 0, C.byref(q), FAKE + 4,
                                     None) == nv.ERR_ALIGN
    assert L.nvfp4_quantize_1d_noise(FAKE, nv.BF16, 16, None, nv.SR, 0, C.byref(q), FAKE,
                                     None) == nv.ERR_SHAPE


def test_qdq_validation(L):
    def call(block=16, fmt=0, rnd=nv.RNE, y=FAKE, ldy=64, amax_in=None, amax_out=FAKE, sums=None,
             x=FAKE, cols=64):
        return L.nvfp4_qdq(x, nv.BF16, 8, cols, 64, block, fmt, amax_in, rnd, 0, y, ldy, amax_out,
                           sums, None)
    assert call(block=12) == nv.ERR_SHAPE
    assert call(fmt=2) == nv.ERR_DTYPE
    assert call(rnd=3) == nv.ERR_DTYPE
    assert call(cols=40, block=32) == nv.ERR_SHAPE
    assert call(y=None) == nv.ERR_NULL
    assert call(ldy=32) == nv.ERR_SHAPE
    assert call(amax_out=None) == nv.ERR_NULL
    assert call(sums=FAKE + 4) == nv.ERR_ALIGN
    assert call(x=FAKE + 2) == nv.ERR_ALIGN


def test_launch_limits_are_rejected(L):
    # shapes whose grids would not fit the launch limits fail validation (nothing is launched)
    big = (1 << 31) - 256
    a, b = _q(big, 64), _q(big, 64)
    assert L.nvfp4_gemm(C.byref(a), C.byref(b), FAKE, nv.F32, big, None) == nv.ERR_SHAPE
    ma, mb = _q(big, 64, layout=nv.MX_1x32), _q(big, 64, layout=nv.MX_1x32)
    assert L.mxfp4_gemm(C.byref(ma), C.byref(mb), FAKE, nv.F32, big, None) == nv.ERR_SHAPE
    T = 512 * 65536                                            # 65536 token blocks of 512
    assert L.nvfp4_hadamard_amax(FAKE, nv.BF16, T, 16, 16, 1, FAKE, None) == nv.ERR_SHAPE
    h = _q(16, T)
    assert L.nvfp4_hadamard_quantize(FAKE, nv.BF16, 16, 1, None, nv.RNE, 0, C.byref(h), None) == nv.ERR_SHAPE



def test_binding_refuses_host_tensors():
    """Host tensors never reach the library (their addresses would fault on the device)."""
    import torch
    x = torch.zeros((16, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        nv._ptr(x)
    with pytest.raises(ValueError):
        nv.quantize_1d(x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without the built HIP library every call raises; there is no fallback path."""
    import torch
    monkeypatch.setattr(nv, "LIB_PATH", str(tmp_path / "libnvfp4.so"))
    monkeypatch.setattr(nv, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        nv.lib()
    with pytest.raises((RuntimeError, ValueError)):
        nv.quantize_1d(torch.zeros((16, 32), dtype=torch.bfloat16))
