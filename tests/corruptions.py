"""Seeded corruptions of coded streams, for the deep-check tests.

Test input generation only: each case edits the bytes of a valid stream (one
written by the CPU oracle) at a place read from its header fields, the way a
damaged file or a bad copy would. Expected results never come from here; the
oracle (and the brute-force restatement) decide what each case is.
"""
import numpy as np


def _u64(s, off):
    return int.from_bytes(bytes(s[off:off + 8]), "little")


def _put_u64(s, off, v):
    s[off:off + 8] = np.frombuffer(int(v % (1 << 64)).to_bytes(8, "little"), np.uint8)


def sections(s):
    """Header fields needed to aim a corruption."""
    return {"nb": _u64(s, 32), "nseg": _u64(s, 40), "meta_off": _u64(s, 56),
            "segoff_off": _u64(s, 64), "payload_off": _u64(s, 72),
            "payload_bytes": _u64(s, 80), "total": _u64(s, 96)}


KINDS = ("width_big", "width_small", "base", "base_max", "segoff_add", "segoff_wrap",
         "segoff_first", "payload")


def corrupt(s, kind, seed):
    """A copy of coded stream s with one seeded corruption of the given kind."""
    rng = np.random.default_rng(seed)
    h = sections(s)
    out = np.array(s, dtype=np.uint8, copy=True)
    nb, nseg = h["nb"], h["nseg"]
    if kind == "width_big":                      # one to three widths above 8
        for _ in range(int(rng.integers(1, 4))):
            out[h["meta_off"] + 2 * int(rng.integers(0, nb)) + 1] = int(rng.integers(9, 256))
    elif kind == "width_small":                  # a width changed within 0..8
        i = int(rng.integers(0, nb))
        w = int(out[h["meta_off"] + 2 * i + 1])
        out[h["meta_off"] + 2 * i + 1] = (w + int(rng.integers(1, 9))) % 9
    elif kind == "base":                         # a base byte replaced
        out[h["meta_off"] + 2 * int(rng.integers(0, nb))] = int(rng.integers(0, 256))
    elif kind == "base_max":                     # a base pushed to 255
        out[h["meta_off"] + 2 * int(rng.integers(0, nb))] = 255
    elif kind == "segoff_add":                   # a stored offset moved by 16..4096
        k = int(rng.integers(0, nseg))
        off = h["segoff_off"] + 8 * k
        _put_u64(out, off, _u64(out, off) + 16 * int(rng.integers(1, 257)))
    elif kind == "segoff_wrap":                  # a stored offset just below 2^64
        k = int(rng.integers(0, nseg))
        _put_u64(out, h["segoff_off"] + 8 * k, (1 << 64) - 16 * int(rng.integers(1, 64)))
    elif kind == "segoff_first":                 # the first offset made nonzero
        _put_u64(out, h["segoff_off"], 16 * int(rng.integers(1, 64)))
    elif kind == "payload":                      # payload bytes overwritten
        for _ in range(int(rng.integers(1, 9))):
            if h["payload_bytes"]:
                out[h["payload_off"] + int(rng.integers(0, h["payload_bytes"]))] = \
                    int(rng.integers(0, 256))
    else:
        raise ValueError(kind)
    return out
