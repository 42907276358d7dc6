"""Lossless block-based fixed-length coding of BF16 weights on MI355X (gfx950).

The GPU library (``libenc.so``, C ABI declared in ``include/enc.h``) does all
the work; :mod:`lossless_weight_compression_amd.enc` is a thin ctypes binding
with the same entry-point names. Importing this package does not load the
library; the first use of a binding name does, and fails loudly if the HIP
library has not been built.
"""
import importlib

_SUBMODULES = ("enc", "synth", "build")


def __getattr__(name):
    if name.startswith("_") or name in _SUBMODULES:
        raise AttributeError(name)
    enc = importlib.import_module(__name__ + ".enc")
    return getattr(enc, name)
