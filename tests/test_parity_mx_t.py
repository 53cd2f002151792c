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
