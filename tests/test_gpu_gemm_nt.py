"""GPU parity of the fused decompress-GEMM for W in linear-layer layout
([N, K] row-major, Y = X . W^T) against the oracle's fp64 product, through
the C ABI.

The oracle computes Y = X . Wt with Wt the transposed (contiguous) copy of
the oracle-decoded W; acceptance per output is |y - Y| <= 1e-4 * sum_k
|x[m,k] * w[n,k]|. One-hot rows of X must reproduce columns of W exactly.
Full size: W 14336 x 4096 (N(0, 0.02), B=512), every output at M = 1, 16
and 128.
"""
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


def bf16_f64(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_nt(orc, X, W):
    """fp64 Y = X . W^T and its bound, W given [N, K]."""
    return orc.gemm_f64(X, np.ascontiguousarray(W.T))


def run_fused(E, X, comp, info, N, ws=None):
    y = E.enc_decompress_gemm_nt(dev(X), comp, info, N, ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def run_dense(E, X, W, ws=None):
    y = E.enc_gemm_dense_nt(dev(X), dev(W), ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_within(y, Y, A, label):
    err = np.abs(y - Y)
    bad = err > TOL * A
    assert not bad.any(), "%s: %d outputs out of tolerance, worst err %g (bound %g)" % (
        label, int(bad.sum()), err[bad].max(), (TOL * A)[bad][np.argmax(err[bad])])


def oracle_stream(E, orc, W, B, pow2=False):
    comp = torch.from_numpy(orc.encode(W.reshape(-1), B, pow2=pow2)).cuda()
    return comp, E.enc_read_info(comp)


@pytest.mark.parametrize("M", [1, 2, 3, 5, 16, 17, 33, 64, 65, 128])
def test_one_hot_rows_exact(E, orc, M):
    N, K = 256, 1024
    W = synth.gaussian_bits((N, K), 0.02, 210, M)
    rng = np.random.default_rng(M)
    X = np.zeros((M, K), np.uint16)
    ks = rng.integers(0, K, M)
    X[np.arange(M), ks] = 0x3F80                     # 1.0
    comp, info = oracle_stream(E, orc, W, 512)
    say("nt one-hot M=%d" % M)
    want = bf16_f64(W)[:, ks].T                     # Y[m, n] = W[n, k_m]
    assert np.array_equal(run_fused(E, X, comp, info, N), want), "fused"
    assert np.array_equal(run_dense(E, X, W), want), "dense"


@pytest.mark.parametrize("B", [128, 256, 512, 1024, 4096])
@pytest.mark.parametrize("M", [1, 2, 5, 16, 33, 70])
def test_block_sizes(E, orc, B, M):
    N, K = 192, 4096
    W = synth.gaussian_bits((N, K), 0.02, 211, B)
    X = synth.gemm_activations(M, K)
    comp, info = oracle_stream(E, orc, W, B)
    Y, A = oracle_nt(orc, X, W)
    say("nt B=%d M=%d" % (B, M))
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused B=%d M=%d" % (B, M))
    assert_within(run_dense(E, X, W), Y, A, "dense B=%d M=%d" % (B, M))


def test_raw_and_pow2_streams(E, orc):
    N, K, M = 128, 512, 7
    X = synth.gemm_activations(M, K)
    Wr = synth.random_bits(N * K, 8, 0, 0x4100).reshape(N, K)   # exponents 0..130: width 8, RAW
    comp, info = oracle_stream(E, orc, Wr, 512)
    assert info.flags == 1
    Y, A = oracle_nt(orc, X, Wr)
    say("nt RAW stream")
    assert_within(run_fused(E, X, comp, info, N), Y, A, "raw")
    W = synth.gaussian_bits((N, K), 0.02, 212, 0)
    comp, info = oracle_stream(E, orc, W, 512, pow2=True)
    assert info.flags == 2
    Y, A = oracle_nt(orc, X, W)
    say("nt power-of-two-width stream")
    assert_within(run_fused(E, X, comp, info, N), Y, A, "pow2")


def test_shape_errors(E, orc):
    W = synth.gaussian_bits((128, 768), 0.02, 213, 0)           # K = 768: not a multiple of 512
    comp, info = oracle_stream(E, orc, W, 512)
    X = dev(synth.gemm_activations(2, 768))
    with pytest.raises(E.EncError) as e:
        E.enc_decompress_gemm_nt(X, comp, info, 128)
    assert e.value.status == -2
    W = synth.gaussian_bits((96, 512), 0.02, 214, 0)            # N = 96: not a multiple of 64
    comp, info = oracle_stream(E, orc, W, 512)
    with pytest.raises(E.EncError) as e:
        E.enc_decompress_gemm_nt(dev(synth.gemm_activations(2, 512)), comp, info, 96)
    assert e.value.status == -2


@pytest.mark.parametrize("M", [1, 16])
def test_full_size_all_outputs(E, orc, M):
    N, K = 14336, 4096
    W = synth.gaussian_bits((N, K), 0.02, 4, 1, outliers=False)
    X = synth.gemm_activations(M, K)
    comp, info = E.enc_compress(dev(W.reshape(-1)), 512)
    say("nt full size M=%d" % M)
    y = run_fused(E, X, comp, info, N)
    Y, A = oracle_nt(orc, X, W)
    assert_within(y, Y, A, "full M=%d" % M)


def test_full_size_m128_all_outputs(E, orc):
    """Every output at M = 128 against the oracle's fp64 product (row ranges
    of X on host threads, the oracle unchanged)."""
    N, K, M = 14336, 4096, 128
    W = synth.gaussian_bits((N, K), 0.02, 4, 1, outliers=False)
    X = synth.gemm_activations(M, K)
    comp, info = E.enc_compress(dev(W.reshape(-1)), 512)
    say("nt full size M=128, all outputs, oracle on %d threads" % oracle_pool.workers())
    y = run_fused(E, X, comp, info, N)
    Y, A = oracle_pool.gemm_f64_rows(orc, X, np.ascontiguousarray(W.T))
    assert_within(y, Y, A, "full M=128")


def test_graph_replay(E):
    N, K, M = 1024, 2048, 9
    W = synth.gaussian_bits((N, K), 0.02, 215, 0)
    X = dev(synth.gemm_activations(M, K))
    comp, info = E.enc_compress(dev(W.reshape(-1)), 512)
    ws = E.gemm_nt_workspace(M, K, N)
    ref = E.enc_decompress_gemm_nt(X, comp, info, N, ws=ws).clone()
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.enc_decompress_gemm_nt(X, comp, info, N, y=y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        E.enc_decompress_gemm_nt(X, comp, info, N, y=y, ws=ws)
    say("nt graph replay")
    for rep in range(3):
        y.fill_(float("nan"))
        ws.fill_(0x55)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), rep


@pytest.mark.parametrize("K", [160, 384, 2080])
@pytest.mark.parametrize("M", [1, 16, 70])
def test_dense_k_steps(E, orc, K, M):
    """The uncompressed [N, K] GEMM for K a multiple of 128 (staged-row
    kernel) and not (fragment kernel)."""
    N = 128
    W = synth.gaussian_bits((N, K), 0.02, 216, K)
    X = synth.gemm_activations(M, K)
    Y, A = oracle_nt(orc, X, W)
    say("nt dense K=%d M=%d" % (K, M))
    assert_within(run_dense(E, X, W), Y, A, "dense K=%d M=%d" % (K, M))


def test_largest_m(E, orc):
    M, N, K = 4096, 128, 512
    W = synth.gaussian_bits((N, K), 0.02, 217, 0)
    rng = np.random.default_rng(4097)
    X = np.zeros((M, K), np.uint16)
    ks = rng.integers(0, K, M)
    X[np.arange(M), ks] = 0x3F80
    comp, info = oracle_stream(E, orc, W, 512)
    say("nt largest M=4096")
    want = bf16_f64(W)[:, ks].T
    assert np.array_equal(run_fused(E, X, comp, info, N), want)
    assert np.array_equal(run_dense(E, X, W), want)


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K,B", [(512, 128), (512, 512), (2048, 256), (4608, 512), (8192, 4096),
                                 (4096, 1024)])
def test_gemv_rows(E, orc, M, K, B):
    """K a multiple of 512, small N: M = 1 runs the workgroup-per-rows GEMV,
    M = 2..4 the staged-row kernel. Every output within the bound, one-hot
    rows of X exact, and the dense twin (same kernels, plain loads) within
    the bound too."""
    N = 192
    W = synth.gaussian_bits((N, K), 0.02, 140, K + B, outliers=True)
    X = synth.gemm_activations(M, K)
    comp, info = oracle_stream(E, orc, W, B)
    say("gemv M=%d K=%d B=%d" % (M, K, B))
    Y, A = oracle_nt(orc, X, W)
    assert_within(run_fused(E, X, comp, info, N), Y, A, "gemv fused")
    assert_within(run_dense(E, X, W), Y, A, "gemv dense")
    # one-hot rows: Y[m, n] = W[n, k_m] exactly
    ks = [(37 * m + 5) % K for m in range(M)]
    Xh = np.zeros((M, K), np.uint16)
    for m, k in enumerate(ks):
        Xh[m, k] = 0x3F80
    y = run_fused(E, Xh, comp, info, N)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], bf16_f64(W[:, k])), (m, k)


@pytest.mark.parametrize("M", [1, 16])
def test_rows_of_mixed_widths(E, orc, M):
    """Rows of W whose blocks have exactly the widths 0, 1, 3, 4, 4, 4, 5, 8
    (in turn, one width per row), B = 512: the waves of the M = 1 GEMV and
    of the staged-row kernel see rows of width 4 only (the nibble split)
    and rows of other widths (bit-field extracts) in the same call."""
    N, K, B = 64, 4096, 512
    rng = np.random.default_rng(143)
    widths = [0, 1, 3, 4, 4, 4, 5, 8]
    W = np.empty((N, K), np.uint16)
    for n in range(N):
        w = widths[n % len(widths)]
        base = 0 if w == 8 else 100
        exps = base + rng.integers(0, 1 << w, K)
        exps.reshape(-1, B)[:, 0] = base                    # every block spans its full range
        exps.reshape(-1, B)[:, 1] = base + (1 << w) - 1
        sm = rng.integers(0, 256, K)
        W[n] = (((sm & 0x80) << 8) | (exps << 7) | (sm & 0x7F)).astype(np.uint16)
    X = synth.gemm_activations(M, K)
    comp, info = oracle_stream(E, orc, W, B)
    assert info.flags == 0
    say("mixed widths M=%d" % M)
    Y, A = oracle_nt(orc, X, W)
    assert_within(run_fused(E, X, comp, info, N), Y, A, "mixed widths")


def test_gemv_raw_and_pow2(E, orc):
    """The M = 1 GEMV on a RAW stream (multiplied from its verbatim values)
    and on a power-of-two-width stream."""
    N, K, M = 64, 1024, 1
    W = synth.random_bits(N * K, 141, 0, 0x4100).reshape(N, K)   # exponents 0..130: width 8, RAW
    X = synth.gemm_activations(M, K)
    comp, info = oracle_stream(E, orc, W, 512)
    assert info.flags == 1
    Y, A = oracle_nt(orc, X, W)
    assert_within(run_fused(E, X, comp, info, N), Y, A, "gemv raw")
    W2 = synth.gaussian_bits((N, K), 0.03, 142, 0)
    comp2, info2 = oracle_stream(E, orc, W2, 512, pow2=True)
    assert info2.flags == 2
    Y2, A2 = oracle_nt(orc, X, W2)
    assert_within(run_fused(E, X, comp2, info2, N), Y2, A2, "gemv pow2")
