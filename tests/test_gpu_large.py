"""A tensor past every 32-bit boundary: 2^32 + 3*2^20 + 13 BF16 values (8.6 GB
in, a ~6.5 GB stream), through the C ABI.

The oracle cannot encode this size in test time, so parity is checked on
what it can compute piece by piece and on properties that hold at any size:
  * the GPU round trip is exact (decode(encode(x)) == x, compared on the GPU);
  * enc_validate accepts the stream;
  * every stored segment offset equals the prefix sum of the padded block
    sizes recomputed on the host (numpy) from the stored widths, and
    payload_bytes equals their total;
  * the {base, width} of sampled blocks (first, around 2^31 and 2^32
    elements, the ragged last one) equal the oracle's for that block's
    values;
  * the oracle's decode_range of the GPU stream at sampled positions (the
    same places) returns the input values.
"""
import sys

import numpy as np
import pytest

from lossless_weight_compression_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

N = (1 << 32) + 3 * (1 << 20) + 13
B = 512


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


def u64(s, off):
    return int.from_bytes(bytes(s[off:off + 8]), "little")


def test_past_32_bit_sizes(E, orc):
    say("large: generating %d values" % N)
    x = synth.gaussian_bits_gpu(N, 0.02, 1)
    say("large: compressing")
    comp, info = E.enc_compress(x, B)
    torch.cuda.synchronize()
    assert info.flags == 0 and info.n_elems == N
    assert info.total_bytes > (1 << 32)
    say("large: stream %d bytes, ratio %.4f" % (info.total_bytes, 2 * N / info.total_bytes))
    chk = E.enc_validate(comp, info)
    assert (chk.kind, chk.index) == (0, 0)
    say("large: decoding")
    out = E.enc_decompress(comp, info)
    torch.cuda.synchronize()
    assert torch.equal(out, x)
    del out
    torch.cuda.empty_cache()

    say("large: host checks")
    s = comp.cpu().numpy()
    nb, nseg = info.n_blocks, info.n_segments
    assert nb == -(-N // B) and nseg == -(-nb // 64)
    meta = s[info.meta_off:info.meta_off + 2 * nb]
    base, w = meta[0::2].astype(np.int64), meta[1::2].astype(np.int64)
    L = np.full(nb, B, np.int64)
    L[-1] = N - (nb - 1) * B
    P = ((w * L + 7) // 8 + 15) // 16 * 16
    starts = np.concatenate([[0], np.cumsum(P)])
    stored = s[info.segoff_off:info.segoff_off + 8 * nseg].view(np.uint64).astype(np.int64)
    assert np.array_equal(stored, starts[0:nb:64])
    assert int(starts[-1]) == info.payload_bytes

    xs = x.view(torch.int16)
    for first in (0, (1 << 31) - 700, (1 << 32) - 1000, N - 5000, N - 13):
        count = min(4096, N - first)
        want = xs[first:first + count].cpu().numpy().view(np.uint16)
        assert np.array_equal(orc.decode_range(s, first, count), want), first
        b0, b1 = first // B, (first + count - 1) // B
        vals = xs[b0 * B:min((b1 + 1) * B, N)].cpu().numpy().view(np.uint16)
        ob, ow = orc.block_params(vals, B)
        assert np.array_equal(base[b0:b1 + 1], ob) and np.array_equal(w[b0:b1 + 1], ow), first
