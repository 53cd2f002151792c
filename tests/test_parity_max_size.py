"""GPU parity on a tensor past 2^32 elements (524544 x 8192 bf16, 8.6 GB): the amax, 1D, dual,
16x16 2D, MXFP4 and dequantize paths index it with 64-bit offsets.  The oracle cannot quantize a
tensor this size in test time, so every check is on outputs it computes independently from a
host copy: the tensor amax over the whole tensor, and sampled rows around element 2^31 and 2^32
(row 262144 starts at element 2^31, row 524288 at 2^32), the first and the last rows, and
sampled 16-feature column blocks for the transposed copies (each depends only on its own
columns).  Round to nearest only: a stochastic-rounding draw depends on the global element
index, which a sampled slice does not carry."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

T, F = 524544, 8192
ROWS = [0, 1, 262143, 262144, 262145, 524287, 524288, T - 1]
COLS = [0, 4096, F - 16]
SIGN = 0x51E4000B


def log(msg):
    print(f"[max-size] {msg}", flush=True)


@pytest.fixture(scope="module")
def big(nv, orc):
    assert T * F > 2 ** 32
    x = W.device_normal_rows((T, F), 20261203)
    torch.cuda.synchronize()
    xh = W.bits(x)                                        # host copy, bf16 bits
    log("tensor generated and copied")
    A = orc.amax(xh)
    log(f"oracle amax {A}")
    yield x, xh, A
    del x
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _rows(t, rows):
    return t[torch.tensor(rows, device=t.device)].cpu().numpy()


def test_amax_and_1d_quantizer_and_dequantize(nv, orc, big):
    x, xh, A = big
    q = nv.quantize_1d(x, nv.RNE)
    torch.cuda.synchronize()
    assert float(q.amax.item()) == A
    o = orc.quantize_1d(np.ascontiguousarray(xh[ROWS]), 0, amax_in=A)
    assert float(q.s_dec.item()) == o["s_dec"]
    np.testing.assert_array_equal(_rows(q.codes, ROWS), o["codes"])
    np.testing.assert_array_equal(_rows(q.scales, ROWS), o["scales"])
    log("1d ok")
    y = nv.dequantize(q, torch.bfloat16)
    np.testing.assert_array_equal(_rows(y.view(torch.int16), ROWS).view(np.uint16),
                                  orc.dequantize(o, len(ROWS), F, out_bf16=True))
    log("dequantize ok")
    del q, y


def test_dual_quantizer(nv, orc, big):
    x, xh, A = big
    At = 4.0 * A                     # at least the transform's amax (|(1/4) H16 D x| <= 4 max|x|)
    q, qt = nv.quantize_dual(x, SIGN, nv.RNE,
                             amax_t_in=torch.tensor([At], dtype=torch.float32, device=x.device))
    torch.cuda.synchronize()
    assert float(q.amax.item()) == A
    o = orc.quantize_1d(np.ascontiguousarray(xh[ROWS]), 0, amax_in=A)
    np.testing.assert_array_equal(_rows(q.codes, ROWS), o["codes"])
    np.testing.assert_array_equal(_rows(q.scales, ROWS), o["scales"])
    for c in COLS:
        ot = orc.hadamard_quantize(np.ascontiguousarray(xh[:, c:c + 16]), SIGN, 0, amax_in=At)
        np.testing.assert_array_equal(qt.codes[c:c + 16].cpu().numpy(), ot["codes"], err_msg=f"cols {c}")
        np.testing.assert_array_equal(qt.scales[c:c + 16].cpu().numpy(), ot["scales"], err_msg=f"cols {c}")
        assert float(qt.s_dec.item()) == ot["s_dec"]
    log("dual ok")
    del q, qt


def test_2d_quantizer(nv, orc, big):
    x, xh, A = big
    q, qt = nv.quantize_2d(x, True)
    torch.cuda.synchronize()
    assert float(q.amax.item()) == A
    for r in (0, 262144, 524288, T - 16):
        o = orc.quantize_2d(np.ascontiguousarray(xh[r:r + 16]), amax_in=A, transposed=False)
        np.testing.assert_array_equal(q.codes[r:r + 16].cpu().numpy(), o["codes"], err_msg=f"rows {r}")
        np.testing.assert_array_equal(q.scales[r // 16:r // 16 + 1].cpu().numpy(), o["scales"])
    for c in COLS:
        o = orc.quantize_2d(np.ascontiguousarray(xh[:, c:c + 16]), amax_in=A, transposed=True)
        np.testing.assert_array_equal(qt.codes[c:c + 16].cpu().numpy(), o["codes_t"], err_msg=f"cols {c}")
        np.testing.assert_array_equal(qt.scales[c // 16:c // 16 + 1].cpu().numpy(), o["scales_t"])
    log("2d ok")
    del q, qt


def test_mx_quantizer(nv, orc, big):
    x, xh, A = big
    q = nv.mx_quantize_1d(x, nv.RNE)
    torch.cuda.synchronize()
    o = orc.mx_quantize_1d(np.ascontiguousarray(xh[ROWS]), 0)
    np.testing.assert_array_equal(_rows(q.codes, ROWS), o["codes"])
    np.testing.assert_array_equal(_rows(q.scales, ROWS), o["scales"])
    log("mx ok")
    del q


def test_gemm_with_operand_past_2gib(nv, orc, big):
    """The same tensor as the A operand of a GEMM (K = 8192: 2.1 GB of codes, rows past the
    2 GiB byte offset) against a 256-row weight: sampled output rows within the GEMM bar of the
    float64 oracle on the oracle's quantization of those rows and of the weight."""
    from gemm_check import assert_gemm_close
    x, xh, A = big
    N = 256
    w = W.weight((N, F), 20261204)
    qa = nv.quantize_1d(x, nv.RNE)
    qb = nv.quantize_1d(w.to(x.device), nv.RNE)
    c = nv.gemm(qa, qb)                                  # fp32 [T x 256]
    torch.cuda.synchronize()
    oa = orc.quantize_1d(np.ascontiguousarray(xh[ROWS]), 0, amax_in=A)
    ob = orc.quantize_1d(W.bits(w), 0)
    ref = orc.gemm_f64(oa, ob, len(ROWS), N, F)
    assert_gemm_close(_rows(c, ROWS), ref, "gemm rows past 2 GiB")
    log("gemm ok")
    del qa, qb, c


def test_gemm_with_output_past_2_31_elements(nv, orc, big):
    """C = x W^T with W 8192 x 8192: 4.3e9 outputs (17 GB in fp32, 8.6 GB in bf16).  Sampled
    output rows (those around output element 2^31 and 2^32 included) meet the GEMM bar in fp32;
    the bf16 output equals the fp32 one rounded to nearest even, and is within one bf16 ulp of
    the oracle's float64 result rounded to bf16 (equal for at least 99.9%)."""
    from gemm_check import assert_gemm_close
    x, xh, A = big
    N = F
    w = W.weight((N, F), 20261205)
    qa = nv.quantize_1d(x, nv.RNE)
    qb = nv.quantize_1d(w.to(x.device), nv.RNE)
    oa = orc.quantize_1d(np.ascontiguousarray(xh[ROWS]), 0, amax_in=A)
    ob = orc.quantize_1d(W.bits(w), 0)
    ref = orc.gemm_f64(oa, ob, len(ROWS), N, F)
    c = nv.gemm(qa, qb)
    torch.cuda.synchronize()
    got = _rows(c, ROWS)
    del c
    assert_gemm_close(got, ref, "fp32 output rows past 2^31 elements")
    cb = nv.gemm(qa, qb, torch.bfloat16)
    torch.cuda.synchronize()
    gb = torch.from_numpy(_rows(cb.view(torch.int16), ROWS)).view(torch.bfloat16)
    del cb
    assert torch.equal(gb.view(torch.int16), torch.from_numpy(got).to(torch.float32)
                       .to(torch.bfloat16).view(torch.int16))
    rb = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16)
    equal = gb.float() == rb.float()
    ulps = torch.where(equal, torch.zeros(equal.shape, dtype=torch.int32),
                       (gb.view(torch.int16).to(torch.int32) - rb.view(torch.int16).to(torch.int32)).abs())
    assert int(ulps.max()) <= 1 and float((ulps == 0).float().mean()) >= 0.999
    log("gemm output ok")
    del qa, qb


def test_mx_gemm_with_operand_past_2gib(nv, orc, big):
    """The MXFP4 comparison GEMM on the same tensor (2.1 GB of codes fetched straight into LDS)
    against a 256-row weight: sampled output rows within the GEMM bar of the oracle."""
    from gemm_check import assert_gemm_close
    x, xh, A = big
    N = 256
    w = W.weight((N, F), 20261206)
    qa = nv.mx_quantize_1d(x, nv.RNE)
    qb = nv.mx_quantize_1d(w.to(x.device), nv.RNE)
    c = nv.mx_gemm(qa, qb)
    torch.cuda.synchronize()
    oa = orc.mx_quantize_1d(np.ascontiguousarray(xh[ROWS]), 0)
    ob = orc.mx_quantize_1d(W.bits(w), 0)
    ref = orc.mx_gemm_f64(oa, ob, len(ROWS), N, F)
    assert_gemm_close(_rows(c, ROWS), ref, "mx gemm rows past 2 GiB")
    log("mx gemm ok")
    del qa, qb, c
