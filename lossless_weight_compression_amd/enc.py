"""ctypes binding of libenc.so (C ABI in include/enc.h), same entry-point names.

Argument marshalling only: every step of compression, decompression and the
fused GEMM runs in the library's gfx950 kernels. torch is used for device
memory (``torch.empty`` on ``cuda``) and for the current HIP stream. If the
library has not been built, the first call raises -- there is no fallback.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libenc.so")

ENC_OK = 0
STATUS_NAMES = {0: "ENC_OK", -1: "ENC_ERR_INVALID_ARG", -2: "ENC_ERR_UNSUPPORTED",
                -3: "ENC_ERR_CAPACITY", -4: "ENC_ERR_BAD_STREAM", -5: "ENC_ERR_SHAPE",
                -6: "ENC_ERR_HIP"}


class EncError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (%d): %s" % (STATUS_NAMES.get(status, "?"), status, message))
        self.status = status


class EncInfo(ctypes.Structure):
    _fields_ = [("version", ctypes.c_uint32), ("dtype", ctypes.c_uint32),
                ("flags", ctypes.c_uint32), ("block_size", ctypes.c_uint32),
                ("n_elems", ctypes.c_uint64), ("n_blocks", ctypes.c_uint64),
                ("n_segments", ctypes.c_uint64), ("sm_off", ctypes.c_uint64),
                ("meta_off", ctypes.c_uint64), ("segoff_off", ctypes.c_uint64),
                ("payload_off", ctypes.c_uint64), ("payload_bytes", ctypes.c_uint64),
                ("raw_off", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}

    def __repr__(self):
        return "EncInfo(%s)" % ", ".join("%s=%s" % kv for kv in self.as_dict().items())


CHECK_NAMES = {0: "ENC_CHECK_OK", 1: "ENC_CHECK_WIDTH", 2: "ENC_CHECK_OFFSETS",
               3: "ENC_CHECK_EXPONENT"}


class EncCheck(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("index", ctypes.c_uint64)]

    def __repr__(self):
        return "EncCheck(%s, index=%d)" % (CHECK_NAMES.get(self.kind, "?"), self.index)


class EncItem(ctypes.Structure):
    _fields_ = [("d_comp", ctypes.c_void_p), ("d_out", ctypes.c_void_p), ("info", EncInfo)]


class EncBatchPlan(ctypes.Structure):
    _fields_ = [("tiles", ctypes.c_uint64), ("wide_tiles", ctypes.c_uint64),
                ("d_table", ctypes.c_void_p), ("count", ctypes.c_int32),
                ("reserved", ctypes.c_uint32)]


class EncCItem(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_void_p), ("n_elems", ctypes.c_uint64),
                ("d_out", ctypes.c_void_p), ("out_capacity", ctypes.c_uint64)]


_VP = ctypes.c_void_p
_U32 = ctypes.c_uint32
_U64 = ctypes.c_uint64
_ST = ctypes.c_int
_INFO_P = ctypes.POINTER(EncInfo)

# name -> (restype, argtypes); exactly the functions include/enc.h declares
SIGNATURES = {
    "enc_compress_bound": (_U64, [_U64]),
    "enc_compress_workspace_bytes": (_U64, [_U64, _U32]),
    "enc_compress": (_ST, [_VP, _U64, _U32, _VP, _U64, _VP, _U64, _VP, _INFO_P]),
    "enc_compress_ex": (_ST, [_VP, _U64, _U32, _U32, _VP, _U64, _VP, _U64, _VP, _INFO_P]),
    "enc_compress_bound_dt": (_U64, [_U64, _U32]),
    "enc_compress_dt": (_ST, [_VP, _U64, _U32, _U32, _U32, _VP, _U64, _VP, _U64, _VP, _INFO_P]),
    "enc_compress_batch_workspace_bytes": (_U64, [ctypes.POINTER(EncCItem), ctypes.c_int, _U32]),
    "enc_compress_batch": (_ST, [ctypes.POINTER(EncCItem), ctypes.c_int, _U32, _U32, _VP, _U64, _VP,
                                 _INFO_P]),
    "enc_compress_batch_dt": (_ST, [ctypes.POINTER(EncCItem), ctypes.c_int, _U32, _U32, _U32, _VP,
                                    _U64, _VP, _INFO_P]),
    "enc_parse_header": (_ST, [_VP, _U64, _U64, _INFO_P]),
    "enc_read_info": (_ST, [_VP, _U64, _VP, _INFO_P]),
    "enc_decompress": (_ST, [_VP, _INFO_P, _VP, _U64, _VP]),
    "enc_batch_table_bytes": (_U64, [ctypes.POINTER(EncItem), ctypes.c_int]),
    "enc_batch_prepare": (_ST, [ctypes.POINTER(EncItem), ctypes.c_int, _VP, _U64, _VP,
                                ctypes.POINTER(EncBatchPlan)]),
    "enc_decompress_batch": (_ST, [_VP, ctypes.c_int, ctypes.POINTER(EncBatchPlan), _VP]),
    "enc_gemm_workspace_bytes": (_U64, [_U32, _U32, _U32, _U32]),
    "enc_decompress_gemm": (_ST, [_VP, _U32, _U32, _VP, _INFO_P, _U32, _VP, _VP, _U64, _VP]),
    "enc_gemm_dense": (_ST, [_VP, _U32, _U32, _VP, _U32, _VP, _VP, _U64, _VP]),
    "enc_gemm_noalloc_scratch_bytes": (_U64, []),
    "enc_decompress_gemm_noalloc": (_ST, [_VP, _U32, _U32, _VP, _INFO_P, _U32, _VP, _VP]),
    "enc_validate_workspace_bytes": (_U64, []),
    "enc_validate": (_ST, [_VP, _INFO_P, _VP, _U64, _VP, ctypes.POINTER(EncCheck)]),
    "enc_gemm_nt_workspace_bytes": (_U64, [_U32, _U32, _U32, _U32]),
    "enc_decompress_gemm_nt": (_ST, [_VP, _U32, _U32, _VP, _INFO_P, _U32, _VP, _VP, _U64, _VP]),
    "enc_gemm_dense_nt": (_ST, [_VP, _U32, _U32, _VP, _U32, _VP, _VP, _U64, _VP]),
    "enc_stream_probe": (_ST, [_VP, _U64, _VP, _U64, _U32, _U32, _VP]),
    "enc_status_string": (ctypes.c_char_p, [_ST]),
    "enc_last_error": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libenc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libenc.so is not built (%s); run "
                               "`python -m lossless_weight_compression_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != ENC_OK:
        raise EncError(status, lib().enc_last_error().decode())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _bits(x):
    """A 16-bit CUDA tensor's storage viewed as int16 (BF16 bit patterns)."""
    import torch
    if x.element_size() != 2:
        raise TypeError("expected a 16-bit tensor of BF16 values or bit patterns")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor")
    return x.view(torch.int16)


BF16, FP16, FP32 = 1, 2, 3           # header element types
ELEM_BYTES = {BF16: 2, FP16: 2, FP32: 4}


def _dtype_of(x, dtype):
    """Header element type of x: given, or float16 -> FP16, float32 -> FP32,
    anything else of 2 bytes (bfloat16, or BF16 bit patterns) -> BF16."""
    import torch
    if dtype is None:
        dtype = {torch.float16: FP16, torch.float32: FP32}.get(x.dtype, BF16)
    if dtype not in ELEM_BYTES:
        raise ValueError("dtype must be 1 (BF16), 2 (FP16) or 3 (FP32)")
    if x.element_size() != ELEM_BYTES[dtype]:
        raise TypeError("a dtype-%d tensor needs %d-byte elements" % (dtype, ELEM_BYTES[dtype]))
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("expected a contiguous CUDA tensor")
    return dtype


def _empty_u8(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------- entry points
def enc_compress_bound(n_elems):
    return int(lib().enc_compress_bound(n_elems))


def enc_compress_workspace_bytes(n_elems, block_size):
    return int(lib().enc_compress_workspace_bytes(n_elems, block_size))


ENC_OPT_POW2_WIDTHS = 1


def enc_compress_bound_dt(n_elems, dtype):
    return int(lib().enc_compress_bound_dt(n_elems, dtype))


def enc_compress(x, block_size=512, out=None, ws=None, stream=None, pow2_widths=False, dtype=None):
    """Compress the tensor x. Returns (stream bytes as a uint8 CUDA tensor
    sliced to the stream size, EncInfo). pow2_widths: ENC_OPT_POW2_WIDTHS.
    BF16 input goes through enc_compress / enc_compress_ex, FP16 and FP32
    input (dtype inferred from x, see _dtype_of) through enc_compress_dt."""
    dtype = _dtype_of(x, dtype)
    if dtype != BF16:
        n = x.numel()
        if out is None:
            out = _empty_u8(enc_compress_bound_dt(n, dtype), x.device)
        if ws is None:
            ws = _empty_u8(enc_compress_workspace_bytes(n, block_size), x.device)
        info = EncInfo()
        _check(lib().enc_compress_dt(_ptr(x), n, dtype, block_size,
                                     ENC_OPT_POW2_WIDTHS if pow2_widths else 0, _ptr(out),
                                     out.numel(), _ptr(ws), ws.numel(), _stream(stream),
                                     ctypes.byref(info)))
        return out[:info.total_bytes], info
    x = _bits(x)
    n = x.numel()
    if out is None:
        out = _empty_u8(enc_compress_bound(n), x.device)
    if ws is None:
        ws = _empty_u8(enc_compress_workspace_bytes(n, block_size), x.device)
    info = EncInfo()
    if pow2_widths:
        _check(lib().enc_compress_ex(_ptr(x), n, block_size, ENC_OPT_POW2_WIDTHS, _ptr(out),
                                     out.numel(), _ptr(ws), ws.numel(), _stream(stream),
                                     ctypes.byref(info)))
    else:
        _check(lib().enc_compress(_ptr(x), n, block_size, _ptr(out), out.numel(), _ptr(ws),
                                  ws.numel(), _stream(stream), ctypes.byref(info)))
    return out[:info.total_bytes], info


def _citems(xs, outs):
    arr = (EncCItem * max(len(xs), 1))()
    for k, (x, out) in enumerate(zip(xs, outs)):
        arr[k].d_in = x.data_ptr()
        arr[k].n_elems = x.numel()
        arr[k].d_out = out.data_ptr()
        arr[k].out_capacity = out.numel() * out.element_size()
    return arr


def enc_compress_batch_workspace_bytes(xs, block_size=512):
    """Workspace bytes enc_compress_batch needs for these BF16 tensors."""
    xs = [_bits(x) for x in xs]
    return lib().enc_compress_batch_workspace_bytes(_citems(xs, xs), len(xs), block_size)


def enc_compress_batch(xs, block_size=512, outs=None, ws=None, stream=None, pow2_widths=False):
    """Compress a list of BF16 tensors with one encoder launch. Returns a list
    of (stream bytes as a uint8 CUDA tensor sliced to its size, EncInfo), each
    byte-identical to enc_compress of the same tensor. outs: uint8 tensors of
    at least enc_compress_bound(n) bytes each (allocated if None)."""
    xs = [_bits(x) for x in xs]
    if not xs:
        return []
    if outs is None:
        outs = [_empty_u8(enc_compress_bound(x.numel()), x.device) for x in xs]
    if len(outs) != len(xs):
        raise ValueError("outs must match xs")
    arr = _citems(xs, outs)
    if ws is None:
        ws = _empty_u8(lib().enc_compress_batch_workspace_bytes(arr, len(xs), block_size),
                       xs[0].device)
    infos = (EncInfo * len(xs))()
    _check(lib().enc_compress_batch(arr, len(xs), block_size,
                                    ENC_OPT_POW2_WIDTHS if pow2_widths else 0, _ptr(ws), ws.numel(),
                                    _stream(stream), infos))
    return [(out[:infos[k].total_bytes], EncInfo.from_buffer_copy(infos[k]))
            for k, out in enumerate(outs)]


def enc_compress_batch_dt(xs, dtype, block_size=512, outs=None, ws=None, stream=None,
                          pow2_widths=False):
    """enc_compress_batch for tensors of one header element type (BF16, FP16
    or FP32; every x must have that type's element size). Each result is
    byte-identical to enc_compress of the same tensor."""
    xs = [x.view(-1) for x in xs]
    if not xs:
        return []
    for x in xs:
        _dtype_of(x, dtype)
    if outs is None:
        outs = [_empty_u8(enc_compress_bound_dt(x.numel(), dtype), x.device) for x in xs]
    if len(outs) != len(xs):
        raise ValueError("outs must match xs")
    arr = _citems(xs, outs)
    if ws is None:
        ws = _empty_u8(lib().enc_compress_batch_workspace_bytes(arr, len(xs), block_size),
                       xs[0].device)
    infos = (EncInfo * len(xs))()
    _check(lib().enc_compress_batch_dt(arr, len(xs), dtype, block_size,
                                       ENC_OPT_POW2_WIDTHS if pow2_widths else 0, _ptr(ws), ws.numel(),
                                       _stream(stream), infos))
    return [(out[:infos[k].total_bytes], EncInfo.from_buffer_copy(infos[k]))
            for k, out in enumerate(outs)]


def enc_parse_header(header, comp_bytes=None):
    """Parse a stream header held in host memory (bytes-like or numpy array)."""
    buf = bytes(memoryview(header).cast("B"))
    if comp_bytes is None:
        comp_bytes = len(buf)
    info = EncInfo()
    cbuf = ctypes.create_string_buffer(buf, len(buf))
    _check(lib().enc_parse_header(cbuf, len(buf), comp_bytes, ctypes.byref(info)))
    return info


def enc_read_info(comp, stream=None):
    info = EncInfo()
    _check(lib().enc_read_info(_ptr(comp), comp.numel() * comp.element_size(), _stream(stream),
                               ctypes.byref(info)))
    return info


def enc_decompress(comp, info, out=None, stream=None):
    """Decode a stream into a CUDA tensor of info.n_elems bit patterns: int16
    for BF16 and FP16 streams, int32 for FP32 streams."""
    import torch
    if out is None:
        tdt = torch.int32 if info.dtype == FP32 else torch.int16
        out = torch.empty(max(info.n_elems, 1), dtype=tdt, device=comp.device)[:info.n_elems]
    _check_out(out, info)
    _check(lib().enc_decompress(_ptr(comp), ctypes.byref(info), _ptr(out), out.numel(),
                                _stream(stream)))
    return out


def _check_out(out, info):
    """The C ABI sees only a pointer and an element count: make sure the
    output tensor holds that many elements of the stream's size."""
    size = ELEM_BYTES.get(info.dtype)
    if size is not None and out.element_size() != size:
        raise TypeError("a dtype-%d stream decodes to %d-byte elements, the output has %d"
                        % (info.dtype, size, out.element_size()))
    if not out.is_contiguous():
        raise ValueError("the output must be contiguous")


def enc_batch_table_bytes(items):
    """Device bytes of the batch table for items: a sequence of (comp,
    EncInfo, out) or of EncInfo."""
    infos = [it if isinstance(it, EncInfo) else it[1] for it in items]
    arr = (EncItem * max(len(infos), 1))()
    for k, info in enumerate(infos):
        arr[k].info = info
    return int(lib().enc_batch_table_bytes(arr, len(infos)))


class BatchTable:
    """A prepared batch: the device table (uint8 CUDA tensor) and the plan
    (launch sizes) enc_batch_prepare filled for it."""

    def __init__(self, table, plan, count):
        self.table, self.plan, self.count = table, plan, count


def enc_batch_prepare(items, table=None, stream=None):
    """items: sequence of (comp tensor, EncInfo, out tensor). Returns a
    BatchTable (table: a device buffer of at least enc_batch_table_bytes)."""
    count = len(items)
    arr = (EncItem * max(count, 1))()
    device = None
    for k, (comp, info, out) in enumerate(items):
        _check_out(out, info)
        if out.numel() != info.n_elems:
            raise ValueError("item %d: output holds %d elements, the stream %d"
                             % (k, out.numel(), info.n_elems))
        arr[k].d_comp = comp.data_ptr()
        arr[k].d_out = out.data_ptr()
        arr[k].info = info
        device = comp.device
    if table is None:
        import torch
        table = _empty_u8(lib().enc_batch_table_bytes(arr, count), device or torch.device("cuda"))
    plan = EncBatchPlan()
    _check(lib().enc_batch_prepare(arr, count, _ptr(table), table.numel(), _stream(stream),
                                   ctypes.byref(plan)))
    return BatchTable(table, plan, count)


def enc_decompress_batch(batch, count=None, stream=None):
    """Decode every item of a BatchTable (count, if given, must match it)."""
    if count is None:
        count = batch.count
    _check(lib().enc_decompress_batch(_ptr(batch.table), count, ctypes.byref(batch.plan),
                                      _stream(stream)))


def enc_gemm_workspace_bytes(M, K, N, block_size=512):
    return int(lib().enc_gemm_workspace_bytes(M, K, N, block_size))


def gemm_workspace(M, K, N, block_size=512, device="cuda"):
    """A zero-filled workspace for enc_decompress_gemm / enc_gemm_dense (it
    starts with arrival counters that must be zero before the first call;
    every call leaves them zero)."""
    import torch
    return torch.zeros(max(enc_gemm_workspace_bytes(M, K, N, block_size), 16), dtype=torch.uint8,
                       device=device)


def enc_decompress_gemm(x, comp, info, N, y=None, ws=None, stream=None):
    """Y[M,N] fp32 = X[M,K] bf16 @ W[K,N], W given compressed."""
    import torch
    x = _bits(x)
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = gemm_workspace(M, K, N, info.block_size, x.device)
    _check(lib().enc_decompress_gemm(_ptr(x), M, K, _ptr(comp), ctypes.byref(info), N, _ptr(y),
                                     _ptr(ws), ws.numel(), _stream(stream)))
    return y


def enc_gemm_noalloc_scratch_bytes():
    return int(lib().enc_gemm_noalloc_scratch_bytes())


def enc_decompress_gemm_noalloc(x, comp, info, N, y=None, stream=None):
    """enc_decompress_gemm with the library's static scratch as workspace."""
    import torch
    x = _bits(x)
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().enc_decompress_gemm_noalloc(_ptr(x), M, K, _ptr(comp), ctypes.byref(info), N,
                                             _ptr(y), _stream(stream)))
    return y


def enc_gemm_dense(x, w, y=None, ws=None, stream=None):
    """Y[M,N] fp32 = X[M,K] bf16 @ W[K,N] bf16 (uncompressed baseline)."""
    import torch
    x = _bits(x)
    w = _bits(w)
    M, K = x.shape
    K2, N = w.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = gemm_workspace(M, K, N, 512, x.device)
    _check(lib().enc_gemm_dense(_ptr(x), M, K, _ptr(w), N, _ptr(y), _ptr(ws), ws.numel(),
                                _stream(stream)))
    return y


def enc_gemm_nt_workspace_bytes(M, K, N, block_size=512):
    return int(lib().enc_gemm_nt_workspace_bytes(M, K, N, block_size))


def gemm_nt_workspace(M, K, N, block_size=512, device="cuda"):
    """A workspace for the [N, K]-layout GEMM entry points (no initialisation needed)."""
    import torch
    return torch.empty(max(enc_gemm_nt_workspace_bytes(M, K, N, block_size), 16), dtype=torch.uint8,
                       device=device)


def enc_decompress_gemm_nt(x, comp, info, N, y=None, ws=None, stream=None):
    """Y[M,N] fp32 = X[M,K] bf16 @ W^T, W [N,K] (linear-layer layout) given compressed."""
    import torch
    x = _bits(x)
    M, K = x.shape
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = gemm_nt_workspace(M, K, N, info.block_size, x.device)
    _check(lib().enc_decompress_gemm_nt(_ptr(x), M, K, _ptr(comp), ctypes.byref(info), N, _ptr(y),
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return y


def enc_gemm_dense_nt(x, w, y=None, ws=None, stream=None):
    """Y[M,N] fp32 = X[M,K] bf16 @ W^T, W [N,K] bf16 uncompressed (baseline)."""
    import torch
    x = _bits(x)
    w = _bits(w)
    M, K = x.shape
    N, K2 = w.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = gemm_nt_workspace(M, K, N, 512, x.device)
    _check(lib().enc_gemm_dense_nt(_ptr(x), M, K, _ptr(w), N, _ptr(y), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    return y


def enc_validate_workspace_bytes():
    return int(lib().enc_validate_workspace_bytes())


def enc_validate(comp, info, ws=None, stream=None):
    """Deep check of a device stream. Returns an EncCheck (kind 0 = valid);
    ENC_ERR_BAD_STREAM is reported through it, other failures raise."""
    if ws is None:
        ws = _empty_u8(enc_validate_workspace_bytes(), comp.device)
    chk = EncCheck()
    st = lib().enc_validate(_ptr(comp), ctypes.byref(info), _ptr(ws), ws.numel(), _stream(stream),
                            ctypes.byref(chk))
    if st != ENC_OK and not (st == -4 and chk.kind != 0):
        _check(st)
    return chk


def enc_stream_probe(src, dst, items_per_thread=1, threads_per_workgroup=256, stream=None):
    """Streaming kernel with the decoder's access shape (measurement helper):
    reads all of `src`, writes all of `dst` (both CUDA tensors)."""
    _check(lib().enc_stream_probe(_ptr(src), src.numel() * src.element_size(), _ptr(dst),
                                  dst.numel() * dst.element_size(), items_per_thread,
                                  threads_per_workgroup, _stream(stream)))


def enc_status_string(status):
    return lib().enc_status_string(status).decode()


def enc_last_error():
    return lib().enc_last_error().decode()
