"""ctypes loader for the C oracle (``enc_oracle.c``).

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the smoke
check and the benchmark's CPU-baseline leg import this module. It builds the
oracle with the host C compiler when the shared library is missing and never
touches the GPU library.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "enc_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f64p = ctypes.POINTER(ctypes.c_double)


def build(force=False):
    """Compile the oracle with gcc (plain -O2, no vector intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-Wextra",
                               "-o", tmp, _SRC])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.orc_exponent.argtypes = [ctypes.c_uint16]
        L.orc_exponent.restype = ctypes.c_uint
        L.orc_signmant.argtypes = [ctypes.c_uint16]
        L.orc_signmant.restype = ctypes.c_uint
        L.orc_join.argtypes = [ctypes.c_uint, ctypes.c_uint]
        L.orc_join.restype = ctypes.c_uint16
        L.orc_bit_width.argtypes = [ctypes.c_uint]
        L.orc_bit_width.restype = ctypes.c_uint
        L.orc_block_payload_bytes.argtypes = [ctypes.c_uint, ctypes.c_uint64]
        L.orc_block_payload_bytes.restype = ctypes.c_uint64
        L.orc_block_params.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, _u8p, _u8p]
        L.orc_block_params.restype = ctypes.c_int64
        L.orc_stream_size.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32]
        L.orc_stream_size.restype = ctypes.c_int64
        L.orc_encode.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, _u8p, ctypes.c_uint64]
        L.orc_encode.restype = ctypes.c_int64
        L.orc_encode_opts.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, _u8p,
                                      ctypes.c_uint64]
        L.orc_encode_opts.restype = ctypes.c_int64
        L.orc_stream_size_opts.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32]
        L.orc_stream_size_opts.restype = ctypes.c_int64
        L.orc_pow2_width.argtypes = [ctypes.c_uint]
        L.orc_pow2_width.restype = ctypes.c_uint
        L.orc_block_params_opts.argtypes = [_u16p, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                            _u8p, _u8p]
        L.orc_block_params_opts.restype = ctypes.c_int64
        L.orc_stream_elements.argtypes = [_u8p, ctypes.c_uint64]
        L.orc_stream_elements.restype = ctypes.c_int64
        L.orc_decode.argtypes = [_u8p, ctypes.c_uint64, _u16p, ctypes.c_uint64]
        L.orc_decode.restype = ctypes.c_int
        L.orc_decode_range.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                       _u16p]
        L.orc_decode_range.restype = ctypes.c_int
        _vp = ctypes.c_void_p
        L.orc_encode_dt.argtypes = [_vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                    ctypes.c_uint32, _u8p, ctypes.c_uint64]
        L.orc_encode_dt.restype = ctypes.c_int64
        L.orc_stream_size_dt.argtypes = [_vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32]
        L.orc_stream_size_dt.restype = ctypes.c_int64
        L.orc_block_params_dt.argtypes = [_vp, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, _u8p, _u8p]
        L.orc_block_params_dt.restype = ctypes.c_int64
        L.orc_decode_dt.argtypes = [_u8p, ctypes.c_uint64, _vp, ctypes.c_uint64]
        L.orc_decode_dt.restype = ctypes.c_int
        L.orc_decode_range_dt.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _vp]
        L.orc_decode_range_dt.restype = ctypes.c_int
        L.orc_stream_dtype.argtypes = [_u8p, ctypes.c_uint64]
        L.orc_stream_dtype.restype = ctypes.c_int64
        for fn in ("orc_exponent_dt", "orc_signmant_dt"):
            getattr(L, fn).argtypes = [ctypes.c_uint32, ctypes.c_uint32]
            getattr(L, fn).restype = ctypes.c_uint32
        L.orc_join_dt.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32]
        L.orc_join_dt.restype = ctypes.c_uint32
        L.orc_validate.argtypes = [_u8p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64)]
        L.orc_validate.restype = ctypes.c_int
        L.orc_gemm_f64.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u16p,
                                   ctypes.c_uint32, _f64p, _f64p]
        L.orc_gemm_f64.restype = None
        L.orc_gemm_f64_cols.argtypes = [_u16p, ctypes.c_uint32, ctypes.c_uint32, _u16p,
                                        ctypes.c_uint32, _u32p, ctypes.c_uint32, _f64p, _f64p]
        L.orc_gemm_f64_cols.restype = None
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _ptr(a, t):
    return a.ctypes.data_as(t)


def _u16(x):
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("expected uint16 BF16 bit patterns")
    return x.reshape(-1)


BF16, FP16, FP32 = 1, 2, 3
_NP = {BF16: np.uint16, FP16: np.uint16, FP32: np.uint32}


def _bits(x, dtype):
    """x as contiguous bit patterns of the element type (uint16 or uint32)."""
    x = np.ascontiguousarray(x)
    if x.dtype != _NP[dtype]:
        raise TypeError("expected %s bit patterns for dtype %d" % (np.dtype(_NP[dtype]).name, dtype))
    return x.reshape(-1)


def exponent_dt(v, dtype):
    return lib().orc_exponent_dt(int(v), dtype)


def signmant_dt(v, dtype):
    return lib().orc_signmant_dt(int(v), dtype)


def join_dt(sm, e, dtype):
    return lib().orc_join_dt(int(sm), int(e), dtype)


def exponent(v):
    return lib().orc_exponent(int(v))


def signmant(v):
    return lib().orc_signmant(int(v))


def join(sm, e):
    return lib().orc_join(int(sm), int(e))


def bit_width(r):
    return lib().orc_bit_width(int(r))


def block_payload_bytes(w, L):
    return lib().orc_block_payload_bytes(int(w), int(L))


def pow2_width(r):
    return lib().orc_pow2_width(int(r))


def block_params(x, B, pow2=False, dtype=BF16):
    """(base[nb], width[nb]) as uint8 arrays."""
    x = _bits(x, dtype)
    nb = -(-x.size // B)
    base = np.zeros(max(nb, 1), np.uint8)
    w = np.zeros(max(nb, 1), np.uint8)
    r = lib().orc_block_params_dt(x.ctypes.data, x.size, dtype, B, 1 if pow2 else 0,
                                  _ptr(base, _u8p), _ptr(w, _u8p))
    if r < 0:
        raise OracleError("block_params failed: %d" % r)
    return base[:nb], w[:nb]


def stream_size(x, B, pow2=False, dtype=BF16):
    x = _bits(x, dtype)
    r = lib().orc_stream_size_dt(x.ctypes.data, x.size, dtype, B, 1 if pow2 else 0)
    if r < 0:
        raise OracleError("stream_size failed: %d" % r)
    return int(r)


def encode(x, B, pow2=False, dtype=BF16):
    """Stream bytes (np.uint8 array) for the bit patterns x (uint16 for BF16
    and FP16, uint32 for FP32) at block size B; pow2: widths rounded up to
    0, 1, 2, 4 or 8 (stream flag 2)."""
    x = _bits(x, dtype)
    size = stream_size(x, B, pow2, dtype)
    out = np.empty(size, np.uint8)
    r = lib().orc_encode_dt(x.ctypes.data, x.size, dtype, B, 1 if pow2 else 0, _ptr(out, _u8p),
                            out.size)
    if r < 0:
        raise OracleError("encode failed: %d" % r)
    assert r == size
    return out


def stream_elements(s):
    s = np.ascontiguousarray(s, dtype=np.uint8)
    return int(lib().orc_stream_elements(_ptr(s, _u8p), s.size))


def stream_dtype(s):
    s = np.ascontiguousarray(s, dtype=np.uint8)
    return int(lib().orc_stream_dtype(_ptr(s, _u8p), s.size))


def decode(s):
    """Decoded bit patterns (uint16 for BF16 / FP16 streams, uint32 for FP32)."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    n = stream_elements(s)
    if n < 0:
        raise OracleError("bad stream: %d" % n)
    out = np.empty(max(n, 1), _NP[stream_dtype(s)])
    r = lib().orc_decode_dt(_ptr(s, _u8p), s.size, out.ctypes.data, n)
    if r != 0:
        raise OracleError("decode failed: %d" % r)
    return out[:n]


def decode_range(s, first, count):
    s = np.ascontiguousarray(s, dtype=np.uint8)
    out = np.empty(max(count, 1), _NP[stream_dtype(s)])
    r = lib().orc_decode_range_dt(_ptr(s, _u8p), s.size, first, count, out.ctypes.data)
    if r != 0:
        raise OracleError("decode_range failed: %d" % r)
    return out[:count]


def validate(s):
    """(kind, index) of the first failing deep condition of a stream whose
    header is consistent: 0 valid, 1 width above 8, 2 wrong stored segment
    offset (index nseg = payload_bytes), 3 exponent above 255."""
    s = np.ascontiguousarray(s, dtype=np.uint8)
    idx = ctypes.c_uint64(0)
    kind = lib().orc_validate(_ptr(s, _u8p), s.size, ctypes.byref(idx))
    if kind < 0:
        raise OracleError("bad header: %d" % kind)
    return int(kind), int(idx.value)


def gemm_f64(X, W):
    """(Y, absbound) in float64 for X [M,K] and W [K,N] given as uint16 BF16 bits."""
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2
    Y = np.empty((M, N), np.float64)
    A = np.empty((M, N), np.float64)
    lib().orc_gemm_f64(_ptr(X, _u16p), M, K, _ptr(W, _u16p), N, _ptr(Y, _f64p), _ptr(A, _f64p))
    return Y, A


def gemm_f64_cols(X, W, cols):
    X = np.ascontiguousarray(X, dtype=np.uint16)
    W = np.ascontiguousarray(W, dtype=np.uint16)
    cols = np.ascontiguousarray(cols, dtype=np.uint32)
    M, K = X.shape
    K2, N = W.shape
    assert K == K2 and (cols < N).all()
    Y = np.empty((M, cols.size), np.float64)
    A = np.empty((M, cols.size), np.float64)
    lib().orc_gemm_f64_cols(_ptr(X, _u16p), M, K, _ptr(W, _u16p), N, _ptr(cols, _u32p), cols.size,
                            _ptr(Y, _f64p), _ptr(A, _f64p))
    return Y, A
