"""The library's launches can be captured in a HIP graph (torch.cuda.graph) and replayed: a
small training step (amax + 1D RNE quantize of X, 2D quantize of W with its transposed copy, the
fprop GEMM; amax + 1D SR quantize of dY and the dgrad GEMM; Hadamard amax + quantize of X and
dY and the wgrad GEMM) captured once and replayed four times, with eager work and outputs
overwritten between replays, gives the eager results bit for bit every time.  No entry point
records a memset; the amax accumulators are zeroed by a kernel."""
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


def test_step_graph_replays_match_eager(nv):
    T, D, O = 512, 256, 384
    x = W.act((T, D), 71).to(DEV)
    w = W.weight((O, D), 72).to(DEV)
    dy = W.grad((T, O), 73).to(DEV)
    Q = nv.QTensor.empty
    qx, qdy = Q(T, D), Q(T, O)
    qw, qwt = Q(O, D, nv.BLK_16x16), Q(D, O, nv.BLK_16x16)
    qxt, qdyt = Q(D, T), Q(O, T)
    y = torch.empty((T, O), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    dw = torch.empty((O, D), dtype=torch.float32, device=DEV)
    sign = 0x51E40007

    def step():
        nv.quantize_1d(x, nv.RNE, out=qx)
        nv.quantize_2d(w, True, out=qw, out_t=qwt)
        nv.gemm(qx, qw, out=y)
        nv.quantize_1d(dy, nv.SR, 0x5EED0071, out=qdy)
        nv.gemm(qdy, qwt, out=dx)
        nv.hadamard_quantize(x, sign, nv.RNE, out=qxt)
        nv.hadamard_quantize(dy, sign, nv.SR, 0x5EED0072, out=qdyt)
        nv.gemm(qdyt, qxt, out=dw)

    def outputs():
        out = []
        for q in (qx, qdy, qw, qwt, qxt, qdyt):
            out += [q.codes, q.scales, q.amax, q.s_dec]
        return out + [y, dx, dw]

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                   # warm-up on a side stream, as capture expects
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in outputs():
            t.fill_(7 if t.dtype == torch.uint8 else -3.0)
        _ = float((x.float() * 2).sum())         # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(), ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
