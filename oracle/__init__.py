"""CPU oracle of the block codec and the compressed-domain reduction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``bit_quantized_all_amd``) never imports it, and the two share no code.

The arithmetic lives in ``qr_oracle.c`` (plain C, IEEE binary32, round to
nearest even); this module only marshals numpy arrays through ctypes.  Values
cross the boundary as raw 16-bit patterns (``uint16``) of fp16 or bf16.

Pages followed: "QuickReduce INT3 quantization and benchmarking on MI355"
(sections Design Highlights; Quantization and Dequantization Paths) and the
"Flash Communication" review (arXiv 2412.04964, key_machinery).
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_BITS = {"int3": 3, "int4": 4, "int8": 8, "asym4": 20, "asym8": 24, "fp4": 36}
DTYPES = {"fp16": 0, "bf16": 1}
TILE = 2048
BLOCK = 32

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)


def _fmt(f):
    return FMT_BITS[f] if isinstance(f, str) else int(f)


def _dt(d):
    return DTYPES[d] if isinstance(d, str) else int(d)


def _ptr(a, t):
    return a.ctypes.data_as(t)


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path=None):
        if path is None:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        self.path = path
        L = ctypes.CDLL(path)
        L.qro_packed_bytes.restype = ctypes.c_size_t
        L.qro_packed_bytes.argtypes = [ctypes.c_int, ctypes.c_size_t]
        L.qro_encode.restype = ctypes.c_int
        L.qro_encode.argtypes = [ctypes.c_int, ctypes.c_int, _u16p, _u8p, ctypes.c_size_t]
        L.qro_decode.restype = ctypes.c_int
        L.qro_decode.argtypes = [ctypes.c_int, ctypes.c_int, _u8p, _u16p, ctypes.c_size_t]
        L.qro_decode_f32.restype = ctypes.c_int
        L.qro_decode_f32.argtypes = [ctypes.c_int, _u8p, _f32p, ctypes.c_size_t]
        L.qro_reduce.restype = ctypes.c_int
        L.qro_reduce.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(_u8p), ctypes.c_int,
                                 _u8p, _u16p, ctypes.c_size_t]
        L.qro_reduce_mixed.restype = ctypes.c_int
        L.qro_reduce_mixed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_u8p),
                                       ctypes.c_int, _u8p, _u16p, ctypes.c_size_t]
        L.qro_group_params.restype = None
        L.qro_group_params.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float, _u16p, _f32p,
                                       ctypes.POINTER(ctypes.c_int)]
        L.qro_block_scale.restype = None
        L.qro_block_scale.argtypes = [ctypes.c_int, ctypes.c_float, _u16p, _f32p]
        L.qro_f16_to_f32.restype = ctypes.c_float
        L.qro_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.qro_f32_to_f16.restype = ctypes.c_uint16
        L.qro_f32_to_f16.argtypes = [ctypes.c_float]
        L.qro_bf16_to_f32.restype = ctypes.c_float
        L.qro_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.qro_f32_to_bf16.restype = ctypes.c_uint16
        L.qro_f32_to_bf16.argtypes = [ctypes.c_float]
        for fn, a, b in (("qro_f32_to_f16_array", _f32p, _u16p), ("qro_f16_to_f32_array", _u16p, _f32p),
                         ("qro_f32_to_bf16_array", _f32p, _u16p), ("qro_bf16_to_f32_array", _u16p, _f32p)):
            getattr(L, fn).restype = None
            getattr(L, fn).argtypes = [a, b, ctypes.c_size_t]
        self.L = L

    # -- sizes ------------------------------------------------------------
    def packed_bytes(self, fmt, n):
        return int(self.L.qro_packed_bytes(_fmt(fmt), n))

    # -- codec --------------------------------------------------------------
    def encode(self, fmt, dtype, x):
        """x: uint16 bit patterns (fp16 or bf16); returns the packed uint8 buffer."""
        x = np.ascontiguousarray(x, dtype=np.uint16).ravel()
        out = np.zeros(self.packed_bytes(fmt, x.size), np.uint8)
        rc = self.L.qro_encode(_fmt(fmt), _dt(dtype), _ptr(x, _u16p), _ptr(out, _u8p), x.size)
        if rc:
            raise ValueError("qro_encode rejected its arguments")
        return out

    def decode(self, fmt, dtype, packed, n):
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        y = np.zeros(n, np.uint16)
        rc = self.L.qro_decode(_fmt(fmt), _dt(dtype), _ptr(packed, _u8p), _ptr(y, _u16p), n)
        if rc:
            raise ValueError("qro_decode rejected its arguments")
        return y

    def decode_f32(self, fmt, packed, n):
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        y = np.zeros(n, np.float32)
        rc = self.L.qro_decode_f32(_fmt(fmt), _ptr(packed, _u8p), _ptr(y, _f32p), n)
        if rc:
            raise ValueError("qro_decode_f32 rejected its arguments")
        return y

    def reduce(self, fmt, dtype, ranks, n, with_output=True):
        """ranks: list of packed uint8 buffers; returns (packed_out, y_out or None)."""
        ranks = [np.ascontiguousarray(r, dtype=np.uint8) for r in ranks]
        arr = (_u8p * len(ranks))(*[_ptr(r, _u8p) for r in ranks])
        out = np.zeros(self.packed_bytes(fmt, n), np.uint8)
        y = np.zeros(n, np.uint16) if with_output else None
        rc = self.L.qro_reduce(_fmt(fmt), _dt(dtype), arr, len(ranks), _ptr(out, _u8p),
                               _ptr(y, _u16p) if with_output else None, n)
        if rc:
            raise ValueError("qro_reduce rejected its arguments")
        return out, y

    def reduce_mixed(self, fmt_in, fmt_out, dtype, ranks, n, with_output=True):
        """Inputs packed in fmt_in, re-encoded sum in fmt_out; returns (packed_out, y_out or None)."""
        ranks = [np.ascontiguousarray(r, dtype=np.uint8) for r in ranks]
        arr = (_u8p * len(ranks))(*[_ptr(r, _u8p) for r in ranks])
        out = np.zeros(self.packed_bytes(fmt_out, n), np.uint8)
        y = np.zeros(n, np.uint16) if with_output else None
        rc = self.L.qro_reduce_mixed(_fmt(fmt_in), _fmt(fmt_out), _dt(dtype), arr, len(ranks),
                                     _ptr(out, _u8p), _ptr(y, _u16p) if with_output else None, n)
        if rc:
            raise ValueError("qro_reduce_mixed rejected its arguments")
        return out, y

    # -- helpers exposed for pinning -----------------------------------------
    def block_scale(self, bits, m):
        d = ctypes.c_uint16()
        e = ctypes.c_float()
        self.L.qro_block_scale(int(bits), float(m), ctypes.byref(d), ctypes.byref(e))
        return d.value, e.value

    def group_params(self, bits, lo, hi):
        d = ctypes.c_uint16()
        e = ctypes.c_float()
        z = ctypes.c_int()
        self.L.qro_group_params(int(bits), float(lo), float(hi), ctypes.byref(d), ctypes.byref(e),
                                ctypes.byref(z))
        return d.value, e.value, z.value

    def _conv(self, fn, x, in_t, out_t, in_p, out_p):
        x = np.ascontiguousarray(x, dtype=in_t).ravel()
        y = np.zeros(x.size, out_t)
        getattr(self.L, fn)(_ptr(x, in_p), _ptr(y, out_p), x.size)
        return y

    def f32_to_f16(self, x):
        return self._conv("qro_f32_to_f16_array", x, np.float32, np.uint16, _f32p, _u16p)

    def f16_to_f32(self, h):
        return self._conv("qro_f16_to_f32_array", h, np.uint16, np.float32, _u16p, _f32p)

    def f32_to_bf16(self, x):
        return self._conv("qro_f32_to_bf16_array", x, np.float32, np.uint16, _f32p, _u16p)

    def bf16_to_f32(self, b):
        return self._conv("qro_bf16_to_f32_array", b, np.uint16, np.float32, _u16p, _f32p)


_DEFAULT = None


def default():
    """The oracle built from ``oracle/qr_oracle.c`` (built on first use if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
