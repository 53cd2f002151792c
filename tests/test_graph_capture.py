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


def test_fused_step_graph_replays_match_eager(nv):
    """The FFN-pair step's calls: one fill of every amax slot, the accumulating dual and weight amax
    passes, the dual-orientation quantizers (RNE and SR), the 2D quantizer, the GEMMs with a split
    last round in a workspace (the wgrad, K = 2048, splits), and the MXFP4 dual quantizer and GEMM,
    captured and replayed."""
    T, D, O = 2048, 256, 384
    x = W.act((T, D), 74).to(DEV)
    w = W.weight((O, D), 75).to(DEV)
    dy = W.grad((T, O), 76).to(DEV)
    Q = nv.QTensor.empty
    qx, qxt, qdy, qdyt = Q(T, D), Q(D, T), Q(T, O), Q(O, T)
    qw, qwt = Q(O, D, nv.BLK_16x16), Q(D, O, nv.BLK_16x16)
    slots = torch.zeros(6, dtype=torch.float32, device=DEV)
    for i, q in enumerate((qx, qxt, qw, qwt, qdy, qdyt)):
        q.amax = slots[i:i + 1]
    mq, mqt = Q(T, D, nv.MX_1x32), Q(D, T, nv.MX_1x32)
    mw, mwt = Q(O, D, nv.MX_1x32), Q(D, O, nv.MX_1x32)
    y = torch.empty((T, O), dtype=torch.bfloat16, device=DEV)
    dx = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    dw = torch.empty((O, D), dtype=torch.float32, device=DEV)
    my = torch.empty((T, O), dtype=torch.float32, device=DEV)
    need = nv.gemm_workspace_size(O, D, T)
    assert need > 0                              # the wgrad's last round is split
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    sign = 0x51E40008

    def step():
        slots.zero_()
        nv.dual_amax_accumulate(x, sign, qx.amax, qxt.amax)
        nv.quantize_dual(x, sign, nv.RNE, 0, 0, amax_in=qx.amax, amax_t_in=qxt.amax, out=qx, out_t=qxt)
        nv.amax_accumulate(w, qw.amax)
        nv.quantize_2d(w, True, amax_in=qw.amax, out=qw, out_t=qwt)
        nv.gemm(qx, qw, out=y, workspace=ws)
        nv.dual_amax_accumulate(dy, sign, qdy.amax, qdyt.amax)
        nv.quantize_dual(dy, sign, nv.SR, 0x5EED0081, 0x5EED0082, amax_in=qdy.amax,
                         amax_t_in=qdyt.amax, out=qdy, out_t=qdyt)
        nv.gemm(qdy, qwt, out=dx, workspace=ws)
        nv.gemm(qdyt, qxt, out=dw, workspace=ws)
        nv.mx_quantize_dual(x, nv.RNE, out=mq, out_t=mqt)
        nv.mx_quantize_dual(w, nv.RNE, out=mw, out_t=mwt)
        nv.mx_gemm(mq, mw, out=my, split=False)

    def outputs():
        out = [slots]
        for q in (qx, qxt, qdy, qdyt, qw, qwt):
            out += [q.codes, q.scales, q.s_dec]
        for q in (mq, mqt, mw, mwt):
            out += [q.codes, q.scales]
        return out + [y, dx, dw, my]

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in outputs():
            t.fill_(7 if t.dtype == torch.uint8 else -3.0)
        _ = float((x.float() * 2).sum())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(), ref)):
            assert torch.equal(a, b), f"replay {r}: output {i} differs"
