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


def _need(t, nbytes, name):
    """The library writes and reads raw device memory: a tensor must hold the
    bytes the call touches (the C ABI cannot check sizes)."""
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _same_device(tensors):
    devs = {t.get_device() for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(devs)}")


def _io(t, dtype, n, name):
    if t.dtype != dtype:
        raise ValueError(f"{name} is {t.dtype}, the call's dtype is {dtype}")
    _need(t, 2 * int(n), name)


def _dt(dtype):
    if dtype not in DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return DTYPES[dtype]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
        raise ValueError(f"{name} must be a contiguous device tensor")
    return ctypes.c_void_p(t.data_ptr())


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
    n = x.numel()
    if packed is None:
        packed = torch.empty(qr_packed_bytes(fmt, n), dtype=torch.uint8, device=x.device)
    _same_device([x, packed])
    _need(packed, qr_packed_bytes(fmt, n), "packed")
    _check("qr_encode", lib().qr_encode(_fmt(fmt), _dt(x.dtype), _dev(x, "x"), _dev(packed, "packed"),
                                        n, _stream(stream)))
    return packed


def qr_decode(fmt, packed, n, dtype, y=None, stream=None):
    """Decode ``n`` values of ``dtype`` from the packed device tensor."""
    if y is None:
        y = torch.empty(n, dtype=dtype, device=packed.device)
    _same_device([packed, y])
    _need(packed, qr_packed_bytes(fmt, n), "packed")
    _io(y, dtype, n, "y")
    _check("qr_decode", lib().qr_decode(_fmt(fmt), _dt(dtype), _dev(packed, "packed"), _dev(y, "y"),
                                        int(n), _stream(stream)))
    return y


def _check_reduce(fmt_in, fmt_out, dtype, ranks, n, packed_out, y_out):
    _same_device(list(ranks) + [packed_out, y_out])
    for r in ranks:
        _need(r, qr_packed_bytes(fmt_in, n), "rank buffer")
    _need(packed_out, qr_packed_bytes(fmt_out, n), "packed_out")
    if y_out is not None:
        _io(y_out, dtype, n, "y_out")


def qr_reduce_compressed(fmt, dtype, ranks, n, packed_out=None, y_out=None, with_output=True,
                         stream=None):
    """Reduce R packed rank buffers; returns (packed_out, y_out or None)."""
    dev = ranks[0].device
    if packed_out is None:
        packed_out = torch.empty(qr_packed_bytes(fmt, n), dtype=torch.uint8, device=dev)
    if y_out is None and with_output:
        y_out = torch.empty(n, dtype=dtype, device=dev)
    _check_reduce(fmt, fmt, dtype, ranks, n, packed_out, y_out)
    arr = (ctypes.c_void_p * len(ranks))(*[_dev(r, "rank").value for r in ranks])
    _check("qr_reduce_compressed",
           lib().qr_reduce_compressed(_fmt(fmt), _dt(dtype), arr, len(ranks), _dev(packed_out, "packed_out"),
                                      _dev(y_out, "y_out") if y_out is not None else None,
                                      int(n), _stream(stream)))
    return packed_out, y_out


def qr_reduce_compressed_mixed(fmt_in, fmt_out, dtype, ranks, n, packed_out=None, y_out=None,
                               with_output=True, stream=None):
    """Inputs packed in fmt_in, re-encoded sum in fmt_out; returns (packed_out, y_out or None)."""
    dev = ranks[0].device
    if packed_out is None:
        packed_out = torch.empty(qr_packed_bytes(fmt_out, n), dtype=torch.uint8, device=dev)
    if y_out is None and with_output:
        y_out = torch.empty(n, dtype=dtype, device=dev)
    _check_reduce(fmt_in, fmt_out, dtype, ranks, n, packed_out, y_out)
    arr = (ctypes.c_void_p * len(ranks))(*[_dev(r, "rank").value for r in ranks])
    _check("qr_reduce_compressed_mixed",
           lib().qr_reduce_compressed_mixed(_fmt(fmt_in), _fmt(fmt_out), _dt(dtype), arr, len(ranks),
                                            _dev(packed_out, "packed_out"),
                                            _dev(y_out, "y_out") if y_out is not None else None,
                                            int(n), _stream(stream)))
    return packed_out, y_out
