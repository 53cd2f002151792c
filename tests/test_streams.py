"""The library keeps no state between calls, so independent work may run concurrently: two host
threads, each driving its own HIP stream through amax, 1D RNE and SR quantizers, the 2D weight
quantizer, the Hadamard quantizer and the GEMMs on its own tensors, give bit for bit what the
same calls give one after the other on one stream, while each thread overwrites its outputs
three times."""
import threading

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


def _chain(nv, x, w, dy, seed):
    T, D = x.shape
    O = w.shape[0]
    Q = nv.QTensor.empty
    qx, qdy = Q(T, D), Q(T, O)
    qw, qwt = Q(O, D, nv.BLK_16x16), Q(D, O, nv.BLK_16x16)
    qxt, qdyt = Q(D, T), Q(O, T)
    nv.quantize_1d(x, nv.RNE, out=qx)
    nv.quantize_2d(w, True, out=qw, out_t=qwt)
    y = nv.gemm(qx, qw, torch.bfloat16)
    nv.quantize_1d(dy, nv.SR, seed, out=qdy)
    dx = nv.gemm(qdy, qwt, torch.bfloat16)
    nv.hadamard_quantize(x, 0x51E40009, nv.RNE, out=qxt)
    nv.hadamard_quantize(dy, 0x51E40009, nv.SR, seed + 1, out=qdyt)
    dw = nv.gemm(qdyt, qxt, torch.float32)
    mx = nv.mx_gemm(nv.mx_quantize_1d(x), nv.mx_quantize_1d(w), torch.float32)
    out = [y, dx, dw, mx]
    for q in (qx, qdy, qw, qwt, qxt, qdyt):
        out += [q.codes, q.scales, q.amax, q.s_dec]
    return out


def test_two_threads_two_streams_match_serial(nv):
    T, D, O = 1024, 512, 768
    inputs = []
    for i in range(2):
        inputs.append((W.act((T, D), 90 + 3 * i).to(DEV), W.weight((O, D), 91 + 3 * i).to(DEV),
                       W.grad((T, O), 92 + 3 * i).to(DEV), 0x5EED0090 + 7 * i))
    torch.cuda.synchronize()
    serial = [[t.clone() for t in _chain(nv, *inp)] for inp in inputs]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in inputs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = [None, None]
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(3):                       # overwrite the outputs a few times
                    res = _chain(nv, *inputs[i])
                results[i] = res
                streams[i].synchronize()
        except Exception as e:                           # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i in range(2):
        for got, exp in zip(results[i], serial[i]):
            assert torch.equal(got.cpu(), exp.cpu())
