"""Thin Python binding of the C ABI in ``include/qr.h``.

Argument marshalling only: every step of the codec and of the reduction runs
in the HIP kernels of ``libqr.so``.  PyTorch supplies device memory and the
current HIP stream.  The library must have been built
(``bit_quantized_all_amd.build``); there is no fallback path.
"""
import ctypes
import functools
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqr.so")

QR_OK, QR_ERR_ARG, QR_ERR_SIZE, QR_ERR_ALIGN, QR_ERR_UNSUPPORTED, QR_ERR_ALIAS, QR_ERR_HIP = range(7)
FORMATS = {"int3": 3, "int4": 4, "int8": 8, "asym4": 20, "asym8": 24, "fp4": 36}
DTYPES = {torch.float16: 0, torch.bfloat16: 1}
TILE_VALUES = 2048
MAX_RANKS = 16

_lib = None


class QRError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {qr_status_string(status)} (status {status})")


def lib():
    """The loaded ``libqr.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with bit_quantized_all_amd.build.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.qr_packed_bytes.restype = sz
        L.qr_packed_bytes.argtypes = [i, sz]
        L.qr_encode.restype = i
        L.qr_encode.argtypes = [i, i, vp, vp, sz, vp]
        L.qr_decode.restype = i
        L.qr_decode.argtypes = [i, i, vp, vp, sz, vp]
        L.qr_reduce_compressed.restype = i
        L.qr_reduce_compressed.argtypes = [i, i, ctypes.POINTER(vp), i, vp, vp, sz, vp]
        L.qr_reduce_compressed_mixed.restype = i
        L.qr_reduce_compressed_mixed.argtypes = [i, i, i, ctypes.POINTER(vp), i, vp, vp, sz, vp]
        L.qr_status_string.restype = ctypes.c_char_p
        L.qr_status_string.argtypes = [i]
        _lib = L
    return _lib


def _fmt(fmt):
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r} (one of {sorted(FORMATS)})")
        return FORMATS[fmt]
    return int(fmt)


def _dt(dtype):
    if dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return DTYPES[dtype]


def _ptr(t, name, nbytes, device=None):
    """Device address of a contiguous device tensor that holds at least
    ``nbytes`` bytes and lives on ``device`` (an index; None takes t's).  The
    library reads and writes raw device memory, so the binding checks here what
    the C ABI cannot: the tensor's kind, size and device."""
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    if device is not None and t.get_device() != device:
        raise ValueError(f"{name} is on device {t.get_device()}, the call's tensors are on device {device}")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")
    return t.data_ptr()


def _io(t, dtype, n, name, device):
    if t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, the call's dtype is {dtype}")
    return _ptr(t, name, 2 * int(n), device)


# The current stream's raw handle without building a torch.cuda.Stream object
# (that costs microseconds per call); the public route where it is missing.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device):
    """HIP stream handle: the given stream, else the current stream of the
    device that holds the call's tensors."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None:
        return _raw_stream(device)
    return torch.cuda.current_stream(device).cuda_stream


def _check(fn, status):
    if status != QR_OK:
        raise QRError(fn, status)


def qr_status_string(status):
    return lib().qr_status_string(int(status)).decode()


@functools.lru_cache(maxsize=1024)
def _packed_bytes(fmt_id, n):
    return int(lib().qr_packed_bytes(fmt_id, n))


def qr_packed_bytes(fmt, n):
    return _packed_bytes(_fmt(fmt), int(n))


def qr_encode(fmt, x, packed=None, stream=None):
    """Encode the fp16/bf16 device tensor ``x``; returns the packed uint8 tensor."""
    fid, n = _fmt(fmt), x.numel()
    pb = _packed_bytes(fid, n)
    if packed is None:
        packed = torch.empty(pb, dtype=torch.uint8, device=x.device)
    xp = _ptr(x, "x", 0)
    dev = x.get_device()
    pp = _ptr(packed, "packed", pb, dev)
    _check("qr_encode", lib().qr_encode(fid, _dt(x.dtype), xp, pp, n, _stream(stream, dev)))
    return packed


def qr_decode(fmt, packed, n, dtype, y=None, stream=None):
    """Decode ``n`` values of ``dtype`` from the packed device tensor."""
    fid, n = _fmt(fmt), int(n)
    if y is None:
        y = torch.empty(n, dtype=dtype, device=packed.device)
    pp = _ptr(packed, "packed", _packed_bytes(fid, n))
    dev = packed.get_device()
    yp = _io(y, dtype, n, "y", dev)
    _check("qr_decode", lib().qr_decode(fid, _dt(dtype), pp, yp, n, _stream(stream, dev)))
    return y


def _reduce(fn, fmt_in, fmt_out, dtype, ranks, n, packed_out, y_out, with_output, stream):
    fi, fo, n = _fmt(fmt_in), _fmt(fmt_out), int(n)
    if not ranks:
        raise ValueError("no rank buffers")
    dev = ranks[0].get_device()
    pin, pout = _packed_bytes(fi, n), _packed_bytes(fo, n)
    if packed_out is None:
        packed_out = torch.empty(pout, dtype=torch.uint8, device=ranks[0].device)
    if y_out is None and with_output:
        y_out = torch.empty(n, dtype=dtype, device=ranks[0].device)
    arr = (ctypes.c_void_p * len(ranks))(*[_ptr(r, "rank buffer", pin, dev) for r in ranks])
    op = _ptr(packed_out, "packed_out", pout, dev)
    yp = _io(y_out, dtype, n, "y_out", dev) if y_out is not None else None
    if fn == "qr_reduce_compressed":
        st = lib().qr_reduce_compressed(fi, _dt(dtype), arr, len(ranks), op, yp, n, _stream(stream, dev))
    else:
        st = lib().qr_reduce_compressed_mixed(fi, fo, _dt(dtype), arr, len(ranks), op, yp, n,
                                              _stream(stream, dev))
    _check(fn, st)
    return packed_out, y_out


def qr_reduce_compressed(fmt, dtype, ranks, n, packed_out=None, y_out=None, with_output=True,
                         stream=None):
    """Reduce R packed rank buffers; returns (packed_out, y_out or None)."""
    return _reduce("qr_reduce_compressed", fmt, fmt, dtype, ranks, n, packed_out, y_out, with_output, stream)


def qr_reduce_compressed_mixed(fmt_in, fmt_out, dtype, ranks, n, packed_out=None, y_out=None,
                               with_output=True, stream=None):
    """Inputs packed in fmt_in, re-encoded sum in fmt_out; returns (packed_out, y_out or None)."""
    return _reduce("qr_reduce_compressed_mixed", fmt_in, fmt_out, dtype, ranks, n, packed_out, y_out,
                   with_output, stream)
