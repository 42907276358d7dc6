"""The deep stream check on the GPU against the CPU oracle, and the library's
behaviour on damaged streams, through the C ABI.

enc_validate must name the same failing condition and the same first failing
block or stored offset as the oracle's validate, on valid streams and on
seeded corruptions of oracle streams. Decoding and the fused GEMM must run to
completion on every damaged stream (their reads stay inside the stream by
construction); on streams the check accepts, decoding must equal the oracle's.
ENC_DEBUG_SYNC must not change any result.
"""
import os
import sys

import numpy as np
import pytest

import corruptions
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


def dev16(x):
    return torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.int16)).cuda()


def dev8(s):
    return torch.from_numpy(np.ascontiguousarray(s, dtype=np.uint8)).cuda()


def test_valid_streams_pass(E, orc):
    cases = [("tiny", synth.tiny(), 512), ("layer.k", synth.layer(names=["k"])["k"], 256),
             ("mixture", synth.stress("mixture"), 1024), ("zeros", synth.stress("zeros"), 128),
             ("uniform16 (RAW)", synth.random_bits(100_000, 5), 512)]
    for name, x, B in cases:
        say("validate valid stream", name, "B=%d" % B)
        comp, info = E.enc_compress(dev16(x), B)
        chk = E.enc_validate(comp, info)
        assert (chk.kind, chk.index) == (0, 0), name
        if x.size <= 1 << 22:
            s = orc.encode(np.ascontiguousarray(x).reshape(-1), B)
            oc = dev8(s)
            chk = E.enc_validate(oc, E.enc_read_info(oc))
            assert (chk.kind, chk.index) == orc.validate(s) == (0, 0), name


@pytest.mark.parametrize("B", [128, 512, 4096])
def test_corruptions_match_oracle(E, orc, B):
    K, N = 384, 4096                         # 1.57M values; N is a multiple of every B
    x = synth.gaussian_bits((K, N), 0.02, 93, B)
    s = orc.encode(x.reshape(-1), B)
    assert s[8] == 0
    X1 = dev16(synth.gemm_activations(1, K))
    X16 = dev16(synth.gemm_activations(16, K)).reshape(16, K)
    X1 = X1.reshape(1, K)
    ws1, ws16 = E.gemm_workspace(1, K, N, B), E.gemm_workspace(16, K, N, B)
    kinds_seen = set()
    for seed, kind in enumerate(corruptions.KINDS * 2):
        b = corruptions.corrupt(s, kind, 7000 + 100 * B + seed)
        want = orc.validate(b)
        kinds_seen.add(want[0])
        say("corruption", kind, "seed", seed, "B=%d" % B, "oracle says", want)
        d = dev8(b)
        info = E.enc_read_info(d)
        chk = E.enc_validate(d, info)
        assert (chk.kind, chk.index) == want, (kind, seed)
        out = E.enc_decompress(d, info)
        E.enc_decompress_gemm(X1, d, info, N, ws=ws1)
        E.enc_decompress_gemm(X16, d, info, N, ws=ws16)
        torch.cuda.synchronize()
        if want[0] == 0:
            assert np.array_equal(out.cpu().numpy().view(np.uint16), orc.decode(b)), (kind, seed)
    assert kinds_seen >= {0, 1, 2, 3}


def test_large_stream_passes(E):
    x = synth.layer(names=["gate"])["gate"]
    say("validate gate 4096x14336 B=512")
    comp, info = E.enc_compress(dev16(x), 512)
    chk = E.enc_validate(comp, info)
    assert chk.kind == 0


def test_debug_sync_changes_nothing(E):
    x = synth.gaussian_bits((512, 2048), 0.02, 94, 0)
    X = dev16(synth.gemm_activations(5, 512)).reshape(5, 512)
    say("ENC_DEBUG_SYNC off/on")
    results = []
    for flag in ("0", "1"):
        os.environ["ENC_DEBUG_SYNC"] = flag
        try:
            comp, info = E.enc_compress(dev16(x), 512)
            out = E.enc_decompress(comp, info)
            o2 = torch.empty_like(out)
            table = E.enc_batch_prepare([(comp, info, o2)])
            E.enc_decompress_batch(table, 1)
            y = E.enc_decompress_gemm(X, comp, info, 2048)
            torch.cuda.synchronize()
            results.append((comp.cpu(), out.cpu(), o2.cpu(), y.cpu()))
        finally:
            os.environ.pop("ENC_DEBUG_SYNC", None)
    for a, b in zip(*results):
        assert torch.equal(a, b)
    assert np.array_equal(results[1][1].numpy().view(np.uint16), x.reshape(-1))


def test_pow2_stream_width_check(E, orc):
    x = synth.gaussian_bits((64, 4096), 0.02, 99, 0)
    s = orc.encode(x.reshape(-1), 512, pow2=True)
    meta = int.from_bytes(bytes(s[56:64]), "little")
    nb = int.from_bytes(bytes(s[32:40]), "little")
    ws = s[meta + 1: meta + 2 * nb: 2]
    i = int(np.flatnonzero(ws == 4)[3])
    b = s.copy(); b[meta + 2 * i + 1] = 3
    for stream in (s, b):
        d = dev8(stream)
        chk = E.enc_validate(d, E.enc_read_info(d))
        assert (chk.kind, chk.index) == orc.validate(stream)
    assert orc.validate(b)[0] == 1


@pytest.mark.parametrize("B", [128, 512])
def test_corruptions_linear_layout_gemm(E, orc, B):
    """The [N, K]-layout GEMM runs to completion on every damaged stream (its
    reads stay inside the stream by construction) and, where the check
    accepts the stream, multiplies exactly the oracle-decoded W."""
    N, K = 256, 4096
    w = synth.gaussian_bits((N, K), 0.02, 95, B)
    s = orc.encode(w.reshape(-1), B)
    assert s[8] == 0
    X = dev16(synth.gemm_activations(16, K)).reshape(16, K)
    one_hot = np.zeros((1, K), np.uint16)
    one_hot[0, 1234] = 0x3F80
    X1 = dev16(one_hot).reshape(1, K)
    ws = E.gemm_nt_workspace(16, K, N, B)
    for seed, kind in enumerate(corruptions.KINDS):
        b = corruptions.corrupt(s, kind, 8100 + 10 * B + seed)
        want = orc.validate(b)
        say("nt corruption", kind, "seed", seed, "B=%d" % B, "oracle says", want)
        d = dev8(b)
        info = E.enc_read_info(d)
        E.enc_decompress_gemm_nt(X, d, info, N, ws=ws)
        y1 = E.enc_decompress_gemm_nt(X1, d, info, N, ws=ws)
        torch.cuda.synchronize()
        if want[0] == 0:
            wd = orc.decode(b).reshape(N, K)
            if ((wd >> 7) & 0xFF == 0xFF).any():
                continue   # a damaged payload made an Inf or NaN: 0 x Inf is NaN
            col = wd[:, 1234].astype(np.uint32) << 16
            assert np.array_equal(y1.cpu().numpy()[0], col.view(np.float32)), (kind, seed)
