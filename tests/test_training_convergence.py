"""End-to-end training through the NVFP4 linear layer: a two-layer GELU MLP student (NVFP4Linear,
fp32 master weights) fitted to a fixed random teacher on seeded synthetic inputs with Adam.  Every
GEMM of the forward and backward passes runs on NVFP4 operands (RNE forward, stochastic rounding on
the gradients, random Hadamard on the weight-gradient operands), so this checks that the
quantized gradients train: the loss must fall far below its start and stay close to the same
student trained in BF16 (the layer's high-precision flag) from the same initialisation, and the
MXFP4 comparison mode must train as well.  Everything is seeded, so the run is deterministic."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda"
D, H, T, STEPS = 256, 1024, 2048, 150


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_bit_quantized_amd as nv
    nv.lib()
    from nvfp4_bit_quantized_amd import linear
    return linear


def _teacher():
    g = torch.Generator(device="cpu").manual_seed(1234)
    w1 = torch.randn(H, D, generator=g) / D ** 0.5
    w2 = torch.randn(D, H, generator=g) / H ** 0.5
    return w1.to(DEV), w2.to(DEV)


def _train(L, mode: str):
    w1t, w2t = _teacher()
    hp = mode == "bf16"
    fmt = "mxfp4" if mode == "mxfp4" else "nvfp4"
    up = L.NVFP4Linear(D, H, high_precision=hp, dtype=torch.float32, seed=11, fmt=fmt)
    down = L.NVFP4Linear(H, D, high_precision=hp, dtype=torch.float32, seed=12, fmt=fmt)
    g = torch.Generator(device="cpu").manual_seed(99)
    with torch.no_grad():
        up.weight.copy_((torch.randn(H, D, generator=g) / D ** 0.5).to(DEV))
        down.weight.copy_((torch.randn(D, H, generator=g) / H ** 0.5).to(DEV))
    opt = torch.optim.Adam(list(up.parameters()) + list(down.parameters()), lr=2e-3)
    gx = torch.Generator(device="cpu").manual_seed(7)
    losses = []
    for _ in range(STEPS):
        x = torch.randn(T, D, generator=gx).to(DEV)
        with torch.no_grad():
            y = torch.nn.functional.gelu(x @ w1t.t()) @ w2t.t()
        if hp:
            out = down(torch.nn.functional.gelu(up(x.bfloat16().float())))
        else:
            out = down(torch.nn.functional.gelu(up(x)))
        loss = torch.mean((out.float() - y) ** 2)
        opt.zero_grad(set_to_none=True)
        loss.backward()
        opt.step()
        losses.append(float(loss.detach()))
    return losses


def test_nvfp4_mlp_trains_like_bf16(L):
    nvl = _train(L, "nvfp4")
    bfl = _train(L, "bf16")
    mxl = _train(L, "mxfp4")
    first, last = nvl[0], sum(nvl[-10:]) / 10
    bf_last, mx_last = sum(bfl[-10:]) / 10, sum(mxl[-10:]) / 10
    print(f"loss start {first:.4f}  NVFP4 {last:.5f}  BF16 {bf_last:.5f}  MXFP4 {mx_last:.5f}")
    assert all(v == v for v in nvl), "NaN in the NVFP4 losses"
    assert last < 0.2 * first, (first, last)
    assert mx_last < 0.2 * first, (first, mx_last)
    # measured: start 0.868, NVFP4 0.1091, BF16 0.1037, MXFP4 0.1101 after 150 steps
    assert last < 1.25 * bf_last, (last, bf_last)
    assert mx_last < 1.25 * bf_last, (mx_last, bf_last)
