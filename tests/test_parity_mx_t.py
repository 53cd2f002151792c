"""GPU parity of the transposing MXFP4 quantizer (x [T x F] -> MXFP4 of x^T [F x T]) against the
CPU oracle's MXFP4 quantizer applied to the transposed matrix: codes and E8M0 scale bytes bit for
bit, RNE and SR (element index feature * T + token)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _same(q, o, what):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.codes.cpu().numpy(), o["codes"], err_msg=f"codes {what}")
    np.testing.assert_array_equal(q.scales.cpu().numpy(), o["scales"], err_msg=f"scales {what}")


SHAPES = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
          ("bf16_act_ragged", lambda: W.act((96, 136), 5)),       # 136 features: 17 groups of 8
          ("bf16_one_block", lambda: W.grad((32, 8), 6)),
          ("bf16_tiles_and_tail", lambda: W.act((544, 4096 + 40), 7)),
          ("fp32_grad", lambda: W.grad((64, 160), 8).float()),
          ("bf16_zero_rows", lambda: torch.zeros((64, 48), dtype=torch.bfloat16))]


@pytest.mark.parametrize("name,make", SHAPES)
@pytest.mark.parametrize("rounding", [0, 1])
def test_mx_quantize_t(nv, orc, name, make, rounding):
    x = make()
    q = nv.mx_quantize_1d_t(x.to(DEV), rounding, seed=0x5EED0005)
    xt = np.ascontiguousarray(W.bits(x).T)
    _same(q, orc.mx_quantize_1d(xt, rounding, 0x5EED0005), f"{name} rnd {rounding}")


def test_mx_quantize_t_strided(nv, orc):
    big = W.act((64, 200), 9)
    x = big[:, 24:24 + 160].contiguous()
    q = nv.mx_quantize_1d_t(big.to(DEV)[:, 24:24 + 160], 1, seed=3)    # ld = 200
    _same(q, orc.mx_quantize_1d(np.ascontiguousarray(W.bits(x).T), 1, 3), "strided")


def test_mx_quantize_t_matches_row_quantizer(nv):
    """On the device too: quantizing x^T row-wise (after a transpose) gives the same bytes."""
    x = W.grad((512, 640), 10).to(DEV)
    for rnd in (0, 1):
        a = nv.mx_quantize_1d_t(x, rnd, seed=77)
        b = nv.mx_quantize_1d(x.t().contiguous(), rnd, seed=77)
        torch.cuda.synchronize()
        assert torch.equal(a.codes, b.codes) and torch.equal(a.scales, b.scales)


def test_mx_quantize_t_ffn_sampled(nv, orc):
    """The FFN down-layer activation gradient dY1 16384 x 20480 (SR): the leading 64 features of
    the transposed copy (whose SR element indices equal the full tensor's) against the oracle."""
    T, FF = W.CFG5["tokens"], W.CFG5["d_ff"]
    x = W.grad((T, FF), W.CFG5["seeds"][5])
    q = nv.mx_quantize_1d_t(x.to(DEV), 1, seed=0x5EED0005)
    torch.cuda.synchronize()
    o = orc.mx_quantize_1d(np.ascontiguousarray(W.bits(x)[:, :64].T), 1, 0x5EED0005)
    np.testing.assert_array_equal(q.codes[:64].cpu().numpy(), o["codes"])
    np.testing.assert_array_equal(q.scales[:64].cpu().numpy(), o["scales"])


DUAL_SHAPES = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
               ("bf16_act_ragged", lambda: W.act((96, 160), 11)),     # partial feature tile
               ("bf16_one_block", lambda: W.grad((32, 32), 12)),
               ("bf16_tiles_and_tail", lambda: W.act((544, 4096 + 32), 13)),
               ("fp32_grad", lambda: W.grad((64, 352), 14).float()),
               ("bf16_zero_rows", lambda: torch.zeros((64, 64), dtype=torch.bfloat16))]


@pytest.mark.parametrize("name,make", DUAL_SHAPES)
@pytest.mark.parametrize("rounding", [0, 1])
def test_mx_quantize_dual(nv, orc, name, make, rounding):
    """One read gives the row-wise MXFP4 copy (element index token * F + feature, seed) and the
    transposed one (feature * T + token, seed_t), each equal to the oracle's MXFP4 quantizer."""
    x = make()
    q, qt = nv.mx_quantize_dual(x.to(DEV), rounding, seed=0x5EED0006, seed_t=0x5EED0007)
    b = W.bits(x)
    _same(q, orc.mx_quantize_1d(b, rounding, 0x5EED0006), f"{name} rows rnd {rounding}")
    _same(qt, orc.mx_quantize_1d(np.ascontiguousarray(b.T), rounding, 0x5EED0007),
          f"{name} transposed rnd {rounding}")


def test_mx_quantize_dual_strided(nv, orc):
    big = W.grad((96, 224), 15)
    x = big[:, 32:32 + 160].contiguous()
    q, qt = nv.mx_quantize_dual(big.to(DEV)[:, 32:32 + 160], 1, seed=5, seed_t=6)    # ld = 224
    b = W.bits(x)
    _same(q, orc.mx_quantize_1d(b, 1, 5), "strided rows")
    _same(qt, orc.mx_quantize_1d(np.ascontiguousarray(b.T), 1, 6), "strided transposed")


def test_mx_quantize_dual_matches_separate_calls(nv):
    """On the device: the fused call writes the bytes of mxfp4_quantize_1d and mxfp4_quantize_1d_t."""
    x = W.act((1024, 1280), 16).to(DEV)
    for rnd in (0, 1):
        q, qt = nv.mx_quantize_dual(x, rnd, seed=41, seed_t=42)
        a = nv.mx_quantize_1d(x, rnd, seed=41)
        at = nv.mx_quantize_1d_t(x, rnd, seed=42)
        torch.cuda.synchronize()
        assert torch.equal(q.codes, a.codes) and torch.equal(q.scales, a.scales)
        assert torch.equal(qt.codes, at.codes) and torch.equal(qt.scales, at.scales)


def test_mx_quantize_dual_ffn_sampled(nv, orc):
    """The FFN down-layer activation gradient dY1 16384 x 20480 (SR): the leading 64 token rows of
    the row-wise copy and the leading 64 feature rows of the transposed copy against the oracle
    (their SR element indices equal the full tensor's)."""
    T, FF = W.CFG5["tokens"], W.CFG5["d_ff"]
    x = W.grad((T, FF), W.CFG5["seeds"][5])
    q, qt = nv.mx_quantize_dual(x.to(DEV), 1, seed=0x5EED0053, seed_t=0x5EED0054)
    torch.cuda.synchronize()
    b = W.bits(x)
    o = orc.mx_quantize_1d(np.ascontiguousarray(b[:64]), 1, 0x5EED0053)
    np.testing.assert_array_equal(q.codes[:64].cpu().numpy(), o["codes"])
    np.testing.assert_array_equal(q.scales[:64].cpu().numpy(), o["scales"])
    ot = orc.mx_quantize_1d(np.ascontiguousarray(b[:, :64].T), 1, 0x5EED0054)
    np.testing.assert_array_equal(qt.codes[:64].cpu().numpy(), ot["codes"])
    np.testing.assert_array_equal(qt.scales[:64].cpu().numpy(), ot["scales"])
