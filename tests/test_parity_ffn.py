"""GPU parity at the FFN linear-pair shapes: up 5120->20480 and down 20480->5120 over 16384
tokens, fprop + dgrad + wgrad in NVFP4 and the MXFP4 comparison.  The tensors are large
(up to 16384x20480), so the oracle checks sampled rows / features: the per-tensor amax is
compared over the whole tensor, then the oracle re-quantizes the sampled rows with that amax and
must match the GPU codes and scales bit-exactly; GEMMs are compared on sampled output rows."""
import numpy as np
import pytest
import torch

import workloads as W
from gemm_check import assert_gemm_close

pytestmark = pytest.mark.gpu

DEV = "cuda"
T, D, FF = W.CFG5["tokens"], W.CFG5["d_model"], W.CFG5["d_ff"]
S_X, S_W1, S_W2, S_H, S_DY2, S_DY1 = W.CFG5["seeds"]
SIGN = 0x51E40005
SR_SEED = 0x5EED0005


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _rows(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, k, replace=False))


def _host_q(q):
    torch.cuda.synchronize()
    d = dict(codes=q.codes.cpu().numpy(), scales=q.scales.cpu().numpy(), layout=q.layout)
    if q.s_dec is not None:
        d["s_dec"] = float(q.s_dec.item())
        d["amax"] = float(q.amax.item())
    return d


def test_ffn_1d_quantizers_sampled(nv, orc):
    """H 16384x20480 (RNE) and dY1 16384x20480 (SR): whole-tensor amax exact; for RNE eight
    sampled rows (a row's codes depend only on the row and the amax), for SR the leading
    64-row block (whose element indices, and so random draws, equal the full tensor's)."""
    for make, seed, rnd in [(W.act, S_H, 0), (W.grad, S_DY1, 1)]:
        x = make((T, FF), seed)
        g = _host_q(nv.quantize_1d(x.to(DEV), rnd, SR_SEED))
        xb = W.bits(x)
        assert g["amax"] == orc.amax(xb)
        blocks = [slice(r, r + 1) for r in _rows(T, 8, seed)] if rnd == 0 else [slice(0, 64)]
        for blk in blocks:
            o = orc.quantize_1d(np.ascontiguousarray(xb[blk]), rnd, SR_SEED, amax_in=g["amax"])
            np.testing.assert_array_equal(g["codes"][blk], o["codes"])
            np.testing.assert_array_equal(g["scales"][blk], o["scales"])
        del x, xb


def test_ffn_2d_quantizer_sampled(nv, orc):
    """W1 20480x5120 with its transposed copy: amax exact, two 16-row tile bands exact."""
    w = W.weight((FF, D), S_W1)
    q, qt = nv.quantize_2d(w.to(DEV), transposed=True)
    g, gt = _host_q(q), _host_q(qt)
    wb = W.bits(w)
    assert g["amax"] == orc.amax(wb)
    for band in (0, 700):
        r0 = band * 16
        o = orc.quantize_2d(np.ascontiguousarray(wb[r0:r0 + 16]), amax_in=g["amax"])
        np.testing.assert_array_equal(g["codes"][r0:r0 + 16], o["codes"])
        np.testing.assert_array_equal(g["scales"][band:band + 1], o["scales"])
        np.testing.assert_array_equal(gt["codes"][:, r0 // 2:r0 // 2 + 8], o["codes_t"])
        np.testing.assert_array_equal(gt["scales"][:, band:band + 1], o["scales_t"])


def test_ffn_hadamard_quantizer_sampled(nv, orc):
    """X 16384x5120 through the RHT (RNE): amax exact, a feature block exact."""
    x = W.act((T, D), S_X)
    g = _host_q(nv.hadamard_quantize(x.to(DEV), SIGN, 0))
    xb = W.bits(x)
    assert g["amax"] == orc.hadamard_amax(xb, SIGN)
    f0 = 1024
    o = orc.hadamard_quantize(np.ascontiguousarray(xb[:, f0:f0 + 64]), SIGN, 0, amax_in=g["amax"])
    np.testing.assert_array_equal(g["codes"][f0:f0 + 64], o["codes"])
    np.testing.assert_array_equal(g["scales"][f0:f0 + 64], o["scales"])


@pytest.fixture(scope="module")
def ffn_operands(nv):
    """Every quantized operand of the pair's forward and backward GEMMs (GPU)."""
    q = {}
    x = W.act((T, D), S_X).to(DEV)
    w1 = W.weight((FF, D), S_W1).to(DEV)
    w2 = W.weight((D, FF), S_W2).to(DEV)
    h = W.act((T, FF), S_H).to(DEV)
    dy2 = W.grad((T, D), S_DY2).to(DEV)
    dy1 = W.grad((T, FF), S_DY1).to(DEV)
    q["x"] = nv.quantize_1d(x)
    q["w1"], q["w1t"] = nv.quantize_2d(w1)
    q["w2"], q["w2t"] = nv.quantize_2d(w2)
    q["h"] = nv.quantize_1d(h)
    q["dy2"] = nv.quantize_1d(dy2, nv.SR, SR_SEED)
    q["dy1"] = nv.quantize_1d(dy1, nv.SR, SR_SEED + 1)
    q["x_t"] = nv.hadamard_quantize(x, SIGN, nv.RNE)
    q["h_t"] = nv.hadamard_quantize(h, SIGN, nv.RNE)
    q["dy2_t"] = nv.hadamard_quantize(dy2, SIGN, nv.SR, SR_SEED + 2)
    q["dy1_t"] = nv.hadamard_quantize(dy1, SIGN, nv.SR, SR_SEED + 3)
    q["mx_x"] = nv.mx_quantize_1d(x)
    q["mx_w1"] = nv.mx_quantize_1d(w1)
    torch.cuda.synchronize()
    del x, w1, w2, h, dy2, dy1
    return q


GEMMS = [  # name, A, B (C = A B^T), output dtype
    ("up_fprop", "x", "w1", torch.bfloat16),       # [T x FF], K = D
    ("down_fprop", "h", "w2", torch.bfloat16),     # [T x D],  K = FF
    ("down_dgrad", "dy2", "w2t", torch.bfloat16),  # [T x FF], K = D
    ("up_dgrad", "dy1", "w1t", torch.bfloat16),    # [T x D],  K = FF
    ("down_wgrad", "dy2_t", "h_t", torch.float32), # [D x FF], K = T
    ("up_wgrad", "dy1_t", "x_t", torch.float32),   # [FF x D], K = T
]


@pytest.mark.parametrize("name,a,b,dt", GEMMS, ids=[g[0] for g in GEMMS])
def test_ffn_gemm_sampled(nv, orc, ffn_operands, name, a, b, dt):
    qa, qb = ffn_operands[a], ffn_operands[b]
    M, N, K = qa.rows, qb.rows, qa.cols
    c = nv.gemm(qa, qb, torch.float32)
    rows = _rows(M, 32, [g[0] for g in GEMMS].index(name) + 11)
    ref = orc.gemm_f64(_host_q(qa), _host_q(qb), M, N, K, rows=rows)
    got = c[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    assert_gemm_close(got, ref, name)
    if dt == torch.bfloat16:
        cb = nv.gemm(qa, qb, torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(cb.view(torch.int16), c.to(torch.bfloat16).view(torch.int16))


def test_ffn_mxfp4_gemm_sampled(nv, orc, ffn_operands):
    qa, qb = ffn_operands["mx_x"], ffn_operands["mx_w1"]
    M, N, K = qa.rows, qb.rows, qa.cols
    c = nv.mx_gemm(qa, qb, torch.float32)
    rows = _rows(M, 32, 5)
    ref = orc.mx_gemm_f64(_host_q(qa), _host_q(qb), M, N, K, rows=rows)
    got = c[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    assert_gemm_close(got, ref, "mxfp4 up fprop")
