"""GPU parity of the fused decompress-GEMM (and its uncompressed twin) against
the oracle's fp64 product, through the C ABI.

Acceptance per output: |y_gpu - y_ref| <= 1e-4 * sum_k |x[m,k] * w[k,n]|,
both reference terms in fp64 from the oracle, with W the oracle-decoded
weight. One-hot rows of X must reproduce rows of W exactly (pins indexing and
layout). Full size: W 4096x14336 (N(0, 0.02), B=512), every output at M in
{1, 16, 128} (M = 128 through the unchanged oracle on host threads).
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


def run_fused(E, X, comp, info, N, ws=None):
    y = E.enc_decompress_gemm(dev(X), comp, info, N, ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def run_dense(E, X, W, ws=None):
    y = E.enc_gemm_dense(dev(X), dev(W), ws=ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def assert_within(y, Y, A, label):
    err = np.abs(y - Y)
    bad = err > TOL * A
    assert not bad.any(), "%s: %d outputs out of tolerance, worst err %g (bound %g)" % (
        label, int(bad.sum()), err[bad].max(), (TOL * A)[bad][np.argmax(err[bad])])


def compress_oracle(orc, W, B):
    """Upload the oracle's stream of W (expected values never come from the GPU)."""
    ref = orc.encode(W.reshape(-1), B)
    comp = torch.from_numpy(ref).cuda()
    return comp, None


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 15, 16, 17, 40, 65, 128, 129, 200])
def test_one_hot_rows_exact(E, orc, M):
    K, N = 256, 1024
    W = synth.gaussian_bits((K, N), 0.02, 200, M)
    rng = np.random.default_rng(M)
    X = np.zeros((M, K), np.uint16)
    ks = rng.integers(0, K, M)
    X[np.arange(M), ks] = 0x3F80                     # 1.0
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    say("one-hot M=%d" % M)
    y = run_fused(E, X, comp, info, N)
    Wf = bf16_f64(W)
    assert np.array_equal(y, Wf[ks]), "fused"
    assert np.array_equal(run_dense(E, X, W), Wf[ks]), "dense"


@pytest.mark.parametrize("B", [128, 256, 512, 1024, 4096])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 16, 33, 130])
def test_block_sizes_small(E, orc, B, M):
    K, N = 520, 4096                                  # K not a multiple of the K ranges
    W = synth.gaussian_bits((K, N), 0.02, 201, B)
    X = synth.gemm_activations(M, K)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), B)).cuda()
    info = E.enc_read_info(comp)
    Y, A = orc.gemm_f64(X, W)
    say("B=%d M=%d" % (B, M))
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused B=%d M=%d" % (B, M))
    assert_within(run_dense(E, X, W), Y, A, "dense B=%d M=%d" % (B, M))


@pytest.mark.parametrize("M", [1, 16, 64])
def test_long_k_ragged_tail(E, orc, M):
    """K = 2056 (a K range ending 8 rows into a 32-row step) and a single
    512-column strip, at B = 256."""
    K, N = 2056, 512
    W = synth.gaussian_bits((K, N), 0.02, 206, M)
    X = synth.gemm_activations(M, K)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 256)).cuda()
    info = E.enc_read_info(comp)
    Y, A = orc.gemm_f64(X, W)
    say("K=%d N=%d M=%d" % (K, N, M))
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused K=%d M=%d" % (K, M))


@pytest.mark.parametrize("M", [2, 16, 100, 130])
def test_long_k_ragged_tail_b512(E, orc, M):
    """K = 2056 at B = 512 (row-uniform kernels: a K range ending 8 rows into
    a 32- or 64-row step), two 512-column strips (four 256-column ones), M
    below, inside and past one 128-row tile."""
    K, N = 2056, 1024
    W = synth.gaussian_bits((K, N), 0.02, 207, M)
    X = synth.gemm_activations(M, K)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    Y, A = orc.gemm_f64(X, W)
    say("K=%d N=%d M=%d B=512" % (K, N, M))
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused K=%d M=%d" % (K, M))
    assert_within(run_dense(E, X, W), Y, A, "dense K=%d M=%d" % (K, M))


def test_raw_weight(E, orc):
    # exponents 1..64 and 129..190 in every block: width 8 everywhere -> RAW
    K, N = 128, 1024
    rng = np.random.default_rng(5)
    exps = np.where(rng.random((K, N)) < 0.5, rng.integers(1, 65, (K, N)),
                    rng.integers(129, 191, (K, N)))
    sm = rng.integers(0, 256, (K, N))
    W = (((sm & 0x80) << 8) | (exps << 7) | (sm & 0x7F)).astype(np.uint16)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    assert info.flags == 1
    for M in (2, 20):
        X = synth.gemm_activations(M, K)
        Y, A = orc.gemm_f64(X, W)
        assert_within(run_fused(E, X, comp, info, N), Y, A, "raw M=%d" % M)


def test_gpu_stream_and_workspace_reuse(E, orc):
    # GPU-compressed W; the same workspace serves consecutive calls (counters
    # are left at zero), results are deterministic, and a smaller M follows
    K, N = 1024, 2048
    W = synth.gaussian_bits((K, N), 0.02, 202, 0)
    comp, info = E.enc_compress(dev(W), 512)
    ws = E.gemm_workspace(64, K, N, 512)
    ys = []
    for M in (64, 64, 24, 2, 1, 1, 2, 64):
        X = synth.gemm_activations(M, K)
        Y, A = orc.gemm_f64(X, W)
        y = run_fused(E, X, comp, info, N, ws=ws)
        assert_within(y, Y, A, "reuse M=%d" % M)
        ys.append(y)
    assert np.array_equal(ys[0], ys[1]) and np.array_equal(ys[0], ys[7])
    assert np.array_equal(ys[4], ys[5]) and np.array_equal(ys[3], ys[6])


@pytest.mark.parametrize("M", [1, 2, 16])
def test_full_size_all_outputs(E, orc, M):
    K, N = 4096, 14336
    W = synth.gemm_weight(K, N)
    X = synth.gemm_activations(M, K)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    say("full size M=%d" % M)
    Y, A = orc.gemm_f64(X, W)
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused full M=%d" % M)
    assert_within(run_dense(E, X, W), Y, A, "dense full M=%d" % M)


def test_full_size_m128_all_outputs(E, orc):
    """Every one of the 128 x 14336 outputs against the oracle's fp64
    product (the unchanged oracle, run on row ranges of X in host threads)."""
    K, N, M = 4096, 14336, 128
    W = synth.gemm_weight(K, N)
    X = synth.gemm_activations(M, K)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    say("full size M=128, all outputs, oracle on %d threads" % oracle_pool.workers())
    Y, A = oracle_pool.gemm_f64_rows(orc, X, W)
    assert_within(run_fused(E, X, comp, info, N), Y, A, "fused M=128")
    assert_within(run_dense(E, X, W), Y, A, "dense M=128")


@pytest.mark.parametrize("M", [1, 5, 16])
def test_pow2_width_stream(E, orc, M):
    """A stream with power-of-two widths (flag 2) multiplies like any other:
    one-hot rows reproduce W exactly, random X within the tolerance."""
    K, N = 256, 2048
    W = synth.gaussian_bits((K, N), 0.02, 203, M)
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512, pow2=True)).cuda()
    info = E.enc_read_info(comp)
    assert info.flags == 2
    rng = np.random.default_rng(M)
    X = np.zeros((M, K), np.uint16)
    ks = rng.integers(0, K, M)
    X[np.arange(M), ks] = 0x3F80
    say("pow2 stream one-hot M=%d" % M)
    assert np.array_equal(run_fused(E, X, comp, info, N), bf16_f64(W)[ks])
    Xr = synth.gemm_activations(M, K)
    Y, A = orc.gemm_f64(Xr, W)
    assert_within(run_fused(E, Xr, comp, info, N), Y, A, "pow2 M=%d" % M)


def test_largest_m(E, orc):
    """M = 4096, the largest the entry point accepts: 32 M tiles of 128 rows;
    one-hot rows reproduce W exactly, the fused and dense paths agree."""
    M, K, N = 4096, 512, 512
    W = synth.gaussian_bits((K, N), 0.02, 204, 0)
    rng = np.random.default_rng(4096)
    X = np.zeros((M, K), np.uint16)
    ks = rng.integers(0, K, M)
    X[np.arange(M), ks] = 0x3F80
    comp = torch.from_numpy(orc.encode(W.reshape(-1), 512)).cuda()
    info = E.enc_read_info(comp)
    say("largest M=4096")
    want = bf16_f64(W)[ks]
    assert np.array_equal(run_fused(E, X, comp, info, N), want)
    assert np.array_equal(run_dense(E, X, W), want)
    with pytest.raises(E.EncError) as e:
        E.enc_decompress_gemm(dev(np.zeros((4097, K), np.uint16)), comp, info, N)
    assert e.value.status == -5
