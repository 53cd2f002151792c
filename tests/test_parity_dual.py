"""GPU parity of the fused dual-orientation quantizer (one read of x, both NVFP4 copies) against
the CPU oracle: the row-wise copy must equal the oracle's 1D quantization and the transposed copy
the oracle's random-Hadamard quantization, bit for bit (codes, scale bytes, amax, s_dec)."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
SIGN = 0x51E40004


@pytest.fixture(scope="module")
def nv():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as m
    m.lib()
    return m


def _same_q(gq, oq, what=""):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gq.codes.cpu().numpy(), oq["codes"], err_msg=f"codes {what}")
    np.testing.assert_array_equal(gq.scales.cpu().numpy(), oq["scales"], err_msg=f"scales {what}")
    assert float(gq.amax.item()) == oq["amax"], what
    assert float(gq.s_dec.item()) == oq["s_dec"], what


SHAPES = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
          ("bf16_act_ragged", lambda: W.act((48, 80), 5)),
          ("bf16_one_chunk", lambda: W.grad((16, 16), 6)),
          ("bf16_tiles_and_tail", lambda: W.act((528, 4096 + 48), 7)),
          ("fp32_grad", lambda: W.grad((96, 160), 8).float()),
          # 256 x 256 tiles: ragged tiles in both directions with whole-word scale stores
          # (F % 64 == 0, T % 64 == 0), and 16 tiles placed XCD by XCD (count % 8 == 0)
          ("bf16_ragged_tiles_word_scales", lambda: W.act((320, 576), 10)),
          ("bf16_sixteen_tiles", lambda: W.grad((2048, 512), 11))]


@pytest.mark.parametrize("name,make", SHAPES)
def test_dual_amax(nv, orc, name, make):
    x = make()
    a, at = nv.dual_amax(x.to(DEV), SIGN)
    torch.cuda.synchronize()
    xb = W.bits(x)
    assert float(a.item()) == orc.amax(xb)
    assert float(at.item()) == orc.hadamard_amax(xb, SIGN)


@pytest.mark.parametrize("name,make", SHAPES)
@pytest.mark.parametrize("rounding", [0, 1])
def test_dual_quantize_small(nv, orc, name, make, rounding):
    x = make()
    q, qt = nv.quantize_dual(x.to(DEV), SIGN, rounding, seed=0x1234, seed_t=0x4321)
    xb = W.bits(x)
    _same_q(q, orc.quantize_1d(xb, rounding=rounding, seed=0x1234), f"{name} rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, rounding, 0x4321), f"{name} transposed")


def test_dual_strided_and_supplied_amax(nv, orc):
    big = W.act((64, 160), 9)
    x = big[:, 16:16 + 128].contiguous()                     # the device view has ld = 160
    xb = W.bits(x)
    dv = big.to(DEV)[:, 16:16 + 128]
    q, qt = nv.quantize_dual(dv, SIGN, 1, seed=3, seed_t=4)
    _same_q(q, orc.quantize_1d(xb, rounding=1, seed=3), "strided rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, 1, 4), "strided transposed")
    a = torch.tensor([3.5], dtype=torch.float32, device=DEV)
    q, qt = nv.quantize_dual(dv, SIGN, 0, amax_in=a)          # transposed amax computed
    _same_q(q, orc.quantize_1d(xb, amax_in=3.5), "amax_in rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, 0, 0), "amax_in transposed")
    at = torch.tensor([0.75], dtype=torch.float32, device=DEV)
    q, qt = nv.quantize_dual(dv, SIGN, 0, amax_t_in=at)        # row-wise amax computed
    _same_q(q, orc.quantize_1d(xb), "amax_t_in rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, 0, 0, amax_in=0.75), "amax_t_in transposed")
    # a supplied amax that lives in the output's own amax slot is used, not recomputed
    qo = nv.QTensor.empty(64, 128, device=DEV)
    qo.amax.fill_(3.5)
    q, qt = nv.quantize_dual(dv, SIGN, 0, amax_in=qo.amax, out=qo)
    _same_q(q, orc.quantize_1d(xb, amax_in=3.5), "aliased amax_in rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, 0, 0), "aliased amax_in transposed")
    q, qt = nv.quantize_dual(dv, SIGN, 0, amax_in=a, amax_t_in=at)
    _same_q(q, orc.quantize_1d(xb, amax_in=3.5), "both given rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, 0, 0, amax_in=0.75), "both given transposed")


def test_dual_empty_and_zero(nv, orc):
    q, qt = nv.quantize_dual(torch.zeros((0, 32), dtype=torch.bfloat16, device=DEV), SIGN)
    torch.cuda.synchronize()
    assert q.amax.item() == 0.0 and q.s_dec.item() == 1.0
    assert qt.amax.item() == 0.0 and qt.s_dec.item() == 1.0
    z = torch.zeros((32, 64), dtype=torch.bfloat16)
    q, qt = nv.quantize_dual(z.to(DEV), SIGN, 1, seed=5, seed_t=6)
    _same_q(q, orc.quantize_1d(W.bits(z), rounding=1, seed=5), "zero rows")
    _same_q(qt, orc.hadamard_quantize(W.bits(z), SIGN, 1, 6), "zero transposed")


@pytest.mark.parametrize("which", ["x", "dy"])
def test_dual_full_size_sampled(nv, orc, which):
    """16384 x 4096 (the wgrad tokens x features): X with RNE, dY with SR (the dgrad and wgrad
    seeds).  Both amaxes over the whole tensor; the leading 64 rows of the row-wise copy and the
    leading 64 features of the transposed copy (whose SR element indices equal the full
    tensor's) against the oracle."""
    if which == "x":
        x, rnd, s1, s2 = W.act((16384, 4096), W.CFG4["seeds"][0]), 0, 0, 0
    else:
        x, rnd, s1, s2 = W.grad((16384, 4096), W.CFG4["seeds"][1]), 1, W.SR_SEED_DGRAD, W.SR_SEED_WGRAD
    q, qt = nv.quantize_dual(x.to(DEV), SIGN, rnd, seed=s1, seed_t=s2)
    torch.cuda.synchronize()
    xb = W.bits(x)
    A, At = orc.amax(xb), orc.hadamard_amax(xb, SIGN)
    assert float(q.amax.item()) == A and float(qt.amax.item()) == At
    o = orc.quantize_1d(np.ascontiguousarray(xb[:64]), rounding=rnd, seed=s1, amax_in=A)
    np.testing.assert_array_equal(q.codes[:64].cpu().numpy(), o["codes"])
    np.testing.assert_array_equal(q.scales[:64].cpu().numpy(), o["scales"])
    ot = orc.hadamard_quantize(np.ascontiguousarray(xb[:, :64]), SIGN, rnd, s2, amax_in=At)
    np.testing.assert_array_equal(qt.codes[:64].cpu().numpy(), ot["codes"])
    np.testing.assert_array_equal(qt.scales[:64].cpu().numpy(), ot["scales"])
    assert float(q.s_dec.item()) == o["s_dec"] and float(qt.s_dec.item()) == ot["s_dec"]
    if rnd == 0:
        # round to nearest depends on the values only: rows and features from the middle and
        # the end of the tensor (other tiles, other XCD ranges) as well
        for r0 in (8192 - 32, 16384 - 64):
            o = orc.quantize_1d(np.ascontiguousarray(xb[r0:r0 + 64]), amax_in=A)
            np.testing.assert_array_equal(q.codes[r0:r0 + 64].cpu().numpy(), o["codes"])
            np.testing.assert_array_equal(q.scales[r0:r0 + 64].cpu().numpy(), o["scales"])
        for f0 in (2048 - 128, 4096 - 64):
            ot = orc.hadamard_quantize(np.ascontiguousarray(xb[:, f0:f0 + 64]), SIGN, 0, 0,
                                       amax_in=At)
            np.testing.assert_array_equal(qt.codes[f0:f0 + 64].cpu().numpy(), ot["codes"])
            np.testing.assert_array_equal(qt.scales[f0:f0 + 64].cpu().numpy(), ot["scales"])


@pytest.mark.parametrize("case", range(8))
def test_dual_random_shapes(nv, orc, case):
    """Seeded random shapes (T % 16 == 0, F % 16 == 0, up to 1200 x 800) through the staged
    quantizer's ragged tiles, both roundings, against the oracle; and the plain Hadamard
    quantizer (the same kernel without its row-wise copy) on F % 8 == 0 shapes."""
    rng = np.random.default_rng(1000 + case)
    T, F = 16 * int(rng.integers(1, 76)), 16 * int(rng.integers(1, 51))
    rounding = case % 2
    x = W.act((T, F), 2000 + case) if case % 4 < 2 else W.grad((T, F), 2000 + case)
    q, qt = nv.quantize_dual(x.to(DEV), SIGN, rounding, seed=case, seed_t=case + 100)
    xb = W.bits(x)
    _same_q(q, orc.quantize_1d(xb, rounding=rounding, seed=case), f"{T}x{F} rows")
    _same_q(qt, orc.hadamard_quantize(xb, SIGN, rounding, case + 100), f"{T}x{F} transposed")
    F8 = 8 * int(rng.integers(1, 101))
    x8 = W.act((T, F8), 3000 + case)
    g = nv.hadamard_quantize(x8.to(DEV), sign_seed=SIGN, rounding=rounding, seed=case)
    _same_q(g, orc.hadamard_quantize(W.bits(x8), SIGN, rounding, case), f"rht {T}x{F8}")
