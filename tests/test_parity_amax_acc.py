"""GPU parity of the accumulating amax calls (nvfp4_amax_accumulate, nvfp4_hadamard_amax_accumulate,
nvfp4_dual_amax_accumulate) against the CPU oracle: starting from 0 they give the oracle's amax bit for bit; they never lower
a caller's value; over several tensors they give the largest amax; an empty tensor changes
nothing."""
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


def _slot(v: float) -> torch.Tensor:
    return torch.full((1,), v, dtype=torch.float32, device=DEV)


CASES = [("fp32_outliers", lambda: W.small_fp32((256, 256), 101)),
         ("bf16_ragged", lambda: W.act((48, 80), 5)),
         ("bf16_grad", lambda: W.grad((512, 136), 6))]


@pytest.mark.parametrize("name,make", CASES)
def test_amax_accumulate_from_zero_is_amax(nv, orc, name, make):
    x = make()
    acc = nv.amax_accumulate(x.to(DEV), _slot(0.0))
    assert acc.item() == orc.amax(W.bits(x)), name
    hacc = nv.hadamard_amax_accumulate(x.to(DEV), 0x51E4, _slot(0.0))
    assert hacc.item() == orc.hadamard_amax(W.bits(x), 0x51E4), name


def test_accumulate_keeps_a_larger_value_and_takes_the_maximum(nv, orc):
    a, b = W.act((64, 96), 11), W.grad((64, 96), 12) * 1000.0
    ma, mb = orc.amax(W.bits(a)), orc.amax(W.bits(b))
    assert ma != mb
    big = 2.0 * max(ma, mb)
    assert nv.amax_accumulate(a.to(DEV), _slot(big)).item() == big
    acc = _slot(0.0)
    nv.amax_accumulate(a.to(DEV), acc)
    nv.amax_accumulate(b.to(DEV), acc)
    assert acc.item() == max(ma, mb)
    ha, hb = orc.hadamard_amax(W.bits(a), 7), orc.hadamard_amax(W.bits(b), 7)
    hacc = _slot(0.0)
    nv.hadamard_amax_accumulate(a.to(DEV), 7, hacc)
    nv.hadamard_amax_accumulate(b.to(DEV), 7, hacc)
    assert hacc.item() == max(ha, hb)
    assert nv.hadamard_amax_accumulate(a.to(DEV), 7, _slot(big)).item() == big


def test_accumulate_empty_leaves_the_slot(nv):
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert nv.amax_accumulate(e, _slot(3.25)).item() == 3.25
    assert nv.hadamard_amax_accumulate(e, 1, _slot(3.25)).item() == 3.25


def test_accumulate_full_size_matches_plain_amax(nv):
    """At the linear-layer step's sizes (8192x4096 and 16384x4096 bf16) the accumulating calls
    from 0 equal the plain calls, which the full-size parity tests pin to the oracle."""
    x = W.act((8192, 4096), 401).to(DEV)
    assert nv.amax_accumulate(x, _slot(0.0)).item() == nv.amax(x).item()
    x4 = W.grad((16384, 4096), 402).to(DEV)
    assert (nv.hadamard_amax_accumulate(x4, 0x51E40004, _slot(0.0)).item()
            == nv.hadamard_amax(x4, 0x51E40004).item())


@pytest.mark.parametrize("name,make", CASES)
def test_dual_amax_accumulate_from_zero(nv, orc, name, make):
    """Both maxima from one read, from 0: the oracle's amax of x and of its Hadamard transform."""
    x = make()
    a, at = nv.dual_amax_accumulate(x.to(DEV), 0x51E4, _slot(0.0), _slot(0.0))
    assert a.item() == orc.amax(W.bits(x)), name
    assert at.item() == orc.hadamard_amax(W.bits(x), 0x51E4), name


def test_dual_amax_accumulate_raises_only(nv, orc):
    a, b = W.act((64, 96), 13), W.grad((64, 96), 14) * 1000.0
    ma, mb = orc.amax(W.bits(a)), orc.amax(W.bits(b))
    ha, hb = orc.hadamard_amax(W.bits(a), 9), orc.hadamard_amax(W.bits(b), 9)
    acc, acc_t = _slot(0.0), _slot(0.0)
    nv.dual_amax_accumulate(a.to(DEV), 9, acc, acc_t)
    nv.dual_amax_accumulate(b.to(DEV), 9, acc, acc_t)
    assert acc.item() == max(ma, mb) and acc_t.item() == max(ha, hb)
    big = 2.0 * max(ma, mb, ha, hb)
    acc, acc_t = nv.dual_amax_accumulate(a.to(DEV), 9, _slot(big), _slot(big))
    assert acc.item() == big and acc_t.item() == big
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    acc, acc_t = nv.dual_amax_accumulate(e, 9, _slot(3.25), _slot(1.5))
    assert acc.item() == 3.25 and acc_t.item() == 1.5


def test_dual_amax_accumulate_full_size(nv):
    """The FFN step's largest activation gradient (16384 x 20480 bf16, streamed) and a smaller one
    (16384 x 5120): from 0 equal to nvfp4_dual_amax, which the full-size tests pin to the oracle."""
    for shape, seed in (((16384, 20480), 506), ((16384, 5120), 505)):
        x = W.grad(shape, seed).to(DEV)
        a, at = nv.dual_amax_accumulate(x, 0x51E40052, _slot(0.0), _slot(0.0))
        b, bt = nv.dual_amax(x, 0x51E40052)
        assert a.item() == b.item() and at.item() == bt.item(), shape
        del x
