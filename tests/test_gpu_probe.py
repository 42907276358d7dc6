"""The streaming probe (a measurement helper beside the codec): every output
item is a copy of a source item, for every workgroup shape, with a ragged
last workgroup; bad shapes are refused before any launch.
"""
import sys

import pytest

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


@pytest.mark.parametrize("threads", [64, 128, 256])
@pytest.mark.parametrize("items", [1, 2, 4])
def test_outputs_are_source_items(E, threads, items):
    # source items are distinct 16-byte values; output 1.32 x longer and not
    # a multiple of one workgroup's run
    ns, nd = 3 * 1024 * 1024 + 17, 4 * 1024 * 1024 + 93
    src = torch.arange(ns * 4, dtype=torch.int32, device="cuda")
    dst = torch.full((nd * 4,), -1, dtype=torch.int32, device="cuda")
    say("probe threads=%d items=%d" % (threads, items))
    E.enc_stream_probe(src, dst, items, threads)
    torch.cuda.synchronize()
    d = dst.view(nd, 4).cpu()
    first = d[:, 0]
    assert bool(((first % 4) == 0).all()), "output items must start on source items"
    idx = first // 4
    assert bool(((idx >= 0) & (idx < ns)).all())
    want = torch.stack([first, first + 1, first + 2, first + 3], dim=1)
    assert torch.equal(d, want), "an output item is not a whole source item"


def test_bad_shapes_refused(E):
    src = torch.zeros(1024, dtype=torch.int32, device="cuda")
    dst = torch.zeros(1024, dtype=torch.int32, device="cuda")
    for items, threads in ((3, 256), (1, 32), (1, 512), (0, 64)):
        with pytest.raises(E.EncError) as e:
            E.enc_stream_probe(src, dst, items, threads)
        assert e.value.status == -1
