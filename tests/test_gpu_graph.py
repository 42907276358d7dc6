"""Entry points captured in a HIP graph (through torch.cuda.CUDAGraph) give,
on every replay, the same bits as eager calls. Eager work (clobbering the
outputs, a synchronisation) runs between the replays. The library records no
memset and no host synchronisation in these paths.
"""
import sys

import numpy as np
import pytest

from lossless_weight_compression_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def E():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_weight_compression_amd import enc
    enc.lib()
    return enc


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).reshape(x.shape).view(np.int16)).cuda()


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_batched_decode_in_graph(E):
    xs = [synth.gaussian_bits((64, 1000), 0.02, 300, 0), synth.random_bits(30_000, 4),
          synth.gaussian_bits((33, 4096), 0.03, 301, 0)]
    items, outs = [], []
    for i, x in enumerate(xs):
        comp, info = E.enc_compress(dev(x.reshape(-1)), (512, 512, 128)[i])
        out = torch.empty(x.size, dtype=torch.int16, device="cuda")
        items.append((comp, info, out))
        outs.append(out)
    table = E.enc_batch_prepare(items)
    say("graph: batched decode")
    g = capture(lambda: E.enc_decompress_batch(table, len(items)))
    for rep in range(3):
        for o in outs:
            o.fill_(rep + 1)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, o in zip(xs, outs):
            assert np.array_equal(o.cpu().numpy().view(np.uint16), x.reshape(-1)), rep


@pytest.mark.parametrize("M", [1, 5, 16, 40])
def test_fused_gemm_in_graph(E, M):
    K, N = 1024, 2048
    W = synth.gaussian_bits((K, N), 0.02, 302, M)
    X = dev(synth.gemm_activations(M, K))
    comp, info = E.enc_compress(dev(W.reshape(-1)), 512)
    ws = E.gemm_workspace(M, K, N)
    ref = E.enc_decompress_gemm(X, comp, info, N, ws=ws).clone()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    say("graph: fused GEMM M=%d" % M)
    g = capture(lambda: E.enc_decompress_gemm(X, comp, info, N, y=y, ws=ws))
    for rep in range(3):
        y.fill_(float("nan"))
        ws[4096:].fill_(0x55)                      # stale scratch (the counters, at the start, stay zero)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep
