"""The C ABI on the host: the library loads, exports every function that
include/qr.h declares, and rejects bad arguments before any HIP call (so these
run without a GPU; no valid compute call is made here)."""
import ctypes
import os
import re

import pytest

import bit_quantized_all_amd as qa
from bit_quantized_all_amd import qr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qr.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qr_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return qa.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == {"qr_packed_bytes", "qr_encode", "qr_decode", "qr_reduce_compressed",
                          "qr_reduce_compressed_mixed", "qr_status_string"}
    for name in names:
        assert hasattr(L, name), name


def test_packed_bytes(L):
    assert L.qr_packed_bytes(3, 2048) == 896
    assert L.qr_packed_bytes(4, 2048) == 1152
    assert L.qr_packed_bytes(8, 2048) == 2176
    assert L.qr_packed_bytes(20, 2048) == 1072   # ASYM4: 1024 codes + 32 scales + 16 zero points
    assert L.qr_packed_bytes(24, 2048) == 2096   # ASYM8: 2048 codes + 32 scales + 16 zero points
    assert L.qr_packed_bytes(20, 2048 * 3) == 1072 * 3
    assert L.qr_packed_bytes(36, 2048 * 5) == 1152 * 5  # FP4: laid out as INT4
    assert L.qr_packed_bytes(4, 2048 * 65536) == 1152 * 65536
    assert L.qr_packed_bytes(4, 0) == 0
    for bad_n in (1, 2047, 2049, 4096 + 32):
        assert L.qr_packed_bytes(4, bad_n) == 0
    for bad_fmt in (0, 2, 5, 6, 16, 19, 21, 23, 25, 28, 32, 35, 37, 40):
        assert L.qr_packed_bytes(bad_fmt, 2048) == 0


def test_status_strings(L):
    for s in range(7):
        assert L.qr_status_string(s) and L.qr_status_string(s) != b"unknown status"
    assert L.qr_status_string(99) == b"unknown status"


# Fake, never-dereferenced device addresses: every call below fails validation.
A = 0x7f0000000000
B = 0x7f0100000000
C = 0x7f0200000000


def enc(L, fmt=4, dt=0, x=A, p=B, n=2048):
    return L.qr_encode(fmt, dt, x, p, n, None)


def dec(L, fmt=4, dt=0, p=A, y=B, n=2048):
    return L.qr_decode(fmt, dt, p, y, n, None)


def red(L, fmt=4, dt=0, ranks=(A,), R=None, out=B, y=C, n=2048):
    arr = (ctypes.c_void_p * max(1, len(ranks)))(*ranks) if ranks is not None else None
    return L.qr_reduce_compressed(fmt, dt, arr, len(ranks) if R is None else R, out, y, n, None)


def test_encode_validation(L):
    assert enc(L, fmt=5) == qr.QR_ERR_UNSUPPORTED
    assert enc(L, dt=2) == qr.QR_ERR_UNSUPPORTED
    assert enc(L, n=2047) == qr.QR_ERR_SIZE
    assert enc(L, n=4096 + 2) == qr.QR_ERR_SIZE
    assert enc(L, x=0) == qr.QR_ERR_ARG
    assert enc(L, p=0) == qr.QR_ERR_ARG
    assert enc(L, x=A + 8) == qr.QR_ERR_ALIGN
    assert enc(L, p=B + 2) == qr.QR_ERR_ALIGN
    # packed starts inside x (x spans 2*n bytes), or x starts inside packed
    assert enc(L, x=A, p=A + 4096 - 16) == qr.QR_ERR_ALIAS
    assert enc(L, x=A + 1152 - 16, p=A) == qr.QR_ERR_ALIAS
    # n == 0 is a size error, whatever the pointers (the size is checked first)
    assert enc(L, n=0, x=0, p=0) == qr.QR_ERR_SIZE
    assert enc(L, n=0) == qr.QR_ERR_SIZE


def test_decode_validation(L):
    assert dec(L, fmt=0) == qr.QR_ERR_UNSUPPORTED
    assert dec(L, dt=-1) == qr.QR_ERR_UNSUPPORTED
    assert dec(L, n=100) == qr.QR_ERR_SIZE
    assert dec(L, p=0) == qr.QR_ERR_ARG
    assert dec(L, y=0) == qr.QR_ERR_ARG
    assert dec(L, y=B + 4) == qr.QR_ERR_ALIGN
    assert dec(L, p=A, y=A + 1024) == qr.QR_ERR_ALIAS
    assert dec(L, n=0, p=0, y=0) == qr.QR_ERR_SIZE
    assert dec(L, n=0) == qr.QR_ERR_SIZE


def test_reduce_validation(L):
    assert red(L, fmt=7) == qr.QR_ERR_UNSUPPORTED
    assert red(L, dt=3) == qr.QR_ERR_UNSUPPORTED
    assert red(L, R=0) == qr.QR_ERR_ARG
    assert red(L, ranks=[A] * 17) == qr.QR_ERR_ARG
    assert red(L, n=2048 + 1) == qr.QR_ERR_SIZE
    assert red(L, ranks=[A, 0]) == qr.QR_ERR_ARG
    assert red(L, out=0) == qr.QR_ERR_ARG
    assert L.qr_reduce_compressed(4, 0, None, 1, B, C, 2048, None) == qr.QR_ERR_ARG
    # overlapping or repeated input ranks are allowed (not checked here: a valid call would launch)
    assert red(L, ranks=[A, A + 8]) == qr.QR_ERR_ALIGN       # ... but must be aligned
    assert red(L, out=B + 8) == qr.QR_ERR_ALIGN
    assert red(L, y=C + 2) == qr.QR_ERR_ALIGN
    assert red(L, ranks=[A, B - 512]) == qr.QR_ERR_ALIAS     # a rank overlaps packed_out
    assert red(L, y=A + 1024) == qr.QR_ERR_ALIAS             # y_out overlaps a rank
    assert red(L, out=C + 2048) == qr.QR_ERR_ALIAS           # outputs overlap each other
    assert red(L, n=0, ranks=[0], out=0, y=0) == qr.QR_ERR_SIZE


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        qa.qr_encode("int4", torch.zeros(2048, dtype=torch.float16), torch.zeros(1152, dtype=torch.uint8))


def redm(L, fi=4, fo=8, dt=0, ranks=(A,), R=None, out=B, y=C, n=2048):
    arr = (ctypes.c_void_p * max(1, len(ranks)))(*ranks)
    return L.qr_reduce_compressed_mixed(fi, fo, dt, arr, len(ranks) if R is None else R, out, y, n, None)


def test_reduce_mixed_validation(L):
    assert redm(L, fi=5) == qr.QR_ERR_UNSUPPORTED
    assert redm(L, fo=2) == qr.QR_ERR_UNSUPPORTED
    assert redm(L, dt=9) == qr.QR_ERR_UNSUPPORTED
    assert redm(L, R=0) == qr.QR_ERR_ARG
    assert redm(L, ranks=[A] * 17) == qr.QR_ERR_ARG
    assert redm(L, n=1000) == qr.QR_ERR_SIZE
    assert redm(L, out=0) == qr.QR_ERR_ARG
    assert redm(L, ranks=[A, A + 4]) == qr.QR_ERR_ALIGN
    # packed_out is sized by fmt_out: an INT8 output (2176 B) starting 2048 B
    # before the INT4 input (1152 B) overlaps it, an INT3 output (896 B) does not
    assert redm(L, fi=4, fo=8, out=A - 2048) == qr.QR_ERR_ALIAS
    assert redm(L, fi=4, fo=8, out=A + 1152 - 16) == qr.QR_ERR_ALIAS
    assert redm(L, fi=8, fo=3, out=A + 2176 - 16) == qr.QR_ERR_ALIAS
    assert redm(L, n=0, ranks=[0], out=0, y=0) == qr.QR_ERR_SIZE


def test_asym_validation(L):
    """Asymmetric formats pass format validation; a symmetric format paired
    with an asymmetric one is unsupported in either direction."""
    assert enc(L, fmt=20, n=2047) == qr.QR_ERR_SIZE
    assert enc(L, fmt=24, p=B + 2) == qr.QR_ERR_ALIGN
    assert dec(L, fmt=20, y=0) == qr.QR_ERR_ARG
    assert red(L, fmt=24, R=17) == qr.QR_ERR_ARG
    for fi, fo in ((4, 20), (20, 4), (8, 24), (24, 3)):
        assert redm(L, fi=fi, fo=fo) == qr.QR_ERR_UNSUPPORTED, (fi, fo)
    # output sized by fmt_out: ASYM8 out (2096 B) 2048 B before an ASYM4 input overlaps it
    assert redm(L, fi=20, fo=24, out=A - 2048) == qr.QR_ERR_ALIAS
    assert redm(L, fi=20, fo=24, out=A + 1072 - 16) == qr.QR_ERR_ALIAS
    assert redm(L, fi=24, fo=20, out=A + 2096 - 16) == qr.QR_ERR_ALIAS
    assert redm(L, fi=20, fo=20, n=0, ranks=[0], out=0, y=0) == qr.QR_ERR_SIZE


def test_fp4_validation(L):
    """FP4 passes format validation; it pairs only with itself in the mixed reduce."""
    assert enc(L, fmt=36, n=2047) == qr.QR_ERR_SIZE
    assert dec(L, fmt=36, p=A + 8) == qr.QR_ERR_ALIGN
    assert red(L, fmt=36, R=0) == qr.QR_ERR_ARG
    for fi, fo in ((4, 36), (36, 4), (36, 20), (24, 36), (36, 8)):
        assert redm(L, fi=fi, fo=fo) == qr.QR_ERR_UNSUPPORTED, (fi, fo)
    assert redm(L, fi=36, fo=36, out=A - 1152 + 16) == qr.QR_ERR_ALIAS
    assert redm(L, fi=36, fo=36, n=0, ranks=[0], out=0, y=0) == qr.QR_ERR_SIZE


def test_too_many_tiles(L):
    """More than QR_MAX_TILES = 2^30 tiles (where a tile index plus one grid
    stride could leave the kernels' int) is a size error, before any HIP call
    (so fake pointers are fine)."""
    n = 2048 * ((1 << 30) + 1)
    assert enc(L, n=n) == qr.QR_ERR_SIZE
    assert dec(L, n=n) == qr.QR_ERR_SIZE
    assert red(L, n=n) == qr.QR_ERR_SIZE
    assert redm(L, n=n) == qr.QR_ERR_SIZE
    assert enc(L, n=2048 * (1 << 30), x=0) == qr.QR_ERR_ARG   # largest accepted count reaches the null check


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback path: with libqr.so absent every call raises instead of
    computing anything elsewhere."""
    import torch

    from bit_quantized_all_amd import qr as Q

    monkeypatch.setattr(Q, "_lib", None)
    monkeypatch.setattr(Q, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libqr.so"))
    Q._packed_bytes.cache_clear()
    try:
        with pytest.raises(RuntimeError, match="missing"):
            Q.lib()
        with pytest.raises(RuntimeError, match="missing"):
            Q.qr_packed_bytes("int4", 2048)
        with pytest.raises(RuntimeError, match="missing"):
            Q.qr_encode("int4", torch.zeros(2048, dtype=torch.float16))
    finally:
        Q._packed_bytes.cache_clear()


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c", "-std=c11"), ("c++", "-std=c++11"), ("c++", "-std=c++17")])
def test_header_compiles_strictly(tmp_path, lang, std):
    """include/qr.h is a plain C header that also compiles as C++ (pedantic,
    warnings as errors), with the enums usable from both."""
    import shutil
    import subprocess

    cc = "gcc" if lang == "c" else "g++"
    if shutil.which(cc) is None:
        pytest.skip(f"{cc} is not installed")
    src = tmp_path / ("h.c" if lang == "c" else "h.cpp")
    src.write_text('#include "qr.h"\n'
                   "int main(void) { qr_format f = QR_INT4; qr_dtype d = QR_BF16; qr_status s = QR_OK;\n"
                   "  return (int)f + (int)d + (int)s - 5 + (int)sizeof(&qr_encode) * 0; }\n")
    r = subprocess.run([cc, std, "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-fsyntax-only", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
