"""The no-allocation fused GEMM (enc_decompress_gemm_noalloc), called through
the C ABI, against enc_decompress_gemm (which takes a caller workspace) and
the oracle's fp64 product: every output within 1e-4 * sum_k |x*w| of the
oracle, and identical to the workspace entry point's (same plan, same
kernels, fixed summation order), on calls in a row that end with a smaller
input; and refusal, before any launch, of a shape whose workspace exceeds
the static scratch."""
import ctypes
import sys

import numpy as np
import pytest

import oracle_pool

from lossless_weight_compression_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = 1e-4


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
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def noalloc(E, X, comp, info, N, y=None):
    x = dev(X)
    M, K = X.shape
    if y is None:
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    st = E.lib().enc_decompress_gemm_noalloc(
        ctypes.c_void_p(x.data_ptr()), M, K, ctypes.c_void_p(comp.data_ptr()), ctypes.byref(info),
        N, ctypes.c_void_p(y.data_ptr()),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise E.EncError(st, E.enc_last_error())
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def with_ws(E, X, comp, info, N):
    y = E.enc_decompress_gemm(dev(X), comp, info, N)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def within(y, Y, A, what):
    err = np.abs(y - Y)
    bad = err > TOL * A
    assert not bad.any(), "%s: %d outputs outside tolerance, worst %g (bound %g)" % (
        what, int(bad.sum()), err.max(), (TOL * A)[np.unravel_index(err.argmax(), err.shape)])


def test_scratch_size(E):
    assert E.lib().enc_gemm_noalloc_scratch_bytes() == 64 << 20


def test_two_calls_full_then_smaller(E, orc):
    """W 4096 x 14336 (B = 512) at M = 128, 16, 1, 1 (the M = 1 kernel reduces
    its K ranges in place through counters in the scratch, which each call
    must leave at zero), then a smaller W; each result against the oracle
    and the workspace entry point."""
    K, N = 4096, 14336
    W = synth.gemm_weight(K, N)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    for M in (128, 16, 1, 1):
        X = synth.gemm_activations(M, K)
        say("noalloc GEMM M=%d K=%d N=%d" % (M, K, N))
        Y, A = oracle_pool.gemm_f64_rows(orc, X, W)
        y0 = noalloc(E, X, comp, info, N)
        y1 = with_ws(E, X, comp, info, N)
        within(y0, Y, A, "noalloc M=%d" % M)
        within(y1, Y, A, "workspace M=%d" % M)
        assert np.array_equal(y0, y1), "noalloc and workspace results differ at M=%d" % M
    K2, N2, M2 = 1024, 2048, 24
    W2 = synth.gaussian_bits((K2, N2), 0.02, 301, 0)
    comp2 = torch.from_numpy(orc.encode(W2.reshape(-1), 512)).cuda()
    info2 = E.enc_read_info(comp2)
    X2 = synth.gemm_activations(M2, K2)
    say("noalloc GEMM, smaller second input M=%d K=%d N=%d" % (M2, K2, N2))
    Y2, A2 = orc.gemm_f64(X2, W2)
    y0 = noalloc(E, X2, comp2, info2, N2)
    y1 = with_ws(E, X2, comp2, info2, N2)
    within(y0, Y2, A2, "noalloc small")
    within(y0, y1, A2, "noalloc vs workspace small")
    assert np.array_equal(y0, y1)   # same plan, same kernels: identical sums


def test_beyond_scratch_is_refused(E, orc):
    """M = 4096 at K = 4096, N = 14336 needs a workspace far above the 64
    MiB scratch: the call fails before any launch and leaves Y untouched."""
    K, N, M = 4096, 14336, 4096
    W = synth.gaussian_bits((K, N), 0.02, 302, 0)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    X = np.zeros((M, K), np.uint16)
    y = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    say("noalloc GEMM beyond the scratch size")
    with pytest.raises(E.EncError) as e:
        noalloc(E, X, comp, info, N, y=y)
    assert e.value.status == -3
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
