"""A second, independent model of the codec and the reduction, in numpy.

Cross-check of the C oracle, not a pin: it restates the same rules, so it
catches slips in either implementation (an index, a shift, a missed branch),
not a shared misreading of the pages.  Nothing here calls the oracle.

Arithmetic is float64 with an explicit rounding to binary32 after every
operation that the codec defines in binary32.  For +, -, * and / of binary32
operands, rounding the float64 result to binary32 gives the correctly rounded
binary32 result (double rounding is harmless when the wider format has at
least 2p + 2 = 50 significand bits; binary64 has 53), so the model takes every
decision in the codec's precision although it computes in float64.
Conversions to binary16 use numpy's float16 cast, conversions to bfloat16
torch's; both round to nearest, ties to even.

Rules restated (pages: "QuickReduce INT3 quantization and benchmarking on
MI355", sections Design Highlights and Quantization and Dequantization Paths;
the "Flash Communication" review, key_machinery and Algorithm 1; the OCP MX
specification for E2M1):

- symmetric b-bit blocks of 32: d = fp16(min(m / 2^(b-1), 65504)),
  e = RN32(1 / d) (0 for d = 0), code = rint(clip(RN32(x e), -Q, Q - 1)) + Q,
  decode (code - Q) d;
- asymmetric b-bit groups of 128: [lo, hi] = [min(x, 0), max(x, 0)],
  s = fp16(min(RN32(RN32(hi - lo) / (2^b - 1)), 65504)), e = RN32(1 / s),
  z = clip(rint(RN32(-lo e)), 0, 2^b - 1), q = clip(rint(RN32(x e)) + z, 0,
  2^b - 1), decode (q - z) s;
- FP4 blocks of 32: d = fp16(min(RN32(m / 6), 65504)), code = nearest E2M1
  value of RN32(x e) with ties to an even mantissa and the sign kept,
  decode value(code) d;
- reduce: decode every rank, sum in rank order with a binary32 rounding after
  each addition, round to the I/O dtype, re-encode, decode.
"""
import numpy as np

import oracle_pins as P

SYM = (3, 4, 8)
ASYM = {20: 4, 24: 8}
FP4 = 36


def r32(a):
    """Round float64 values to binary32 (overflow gives +-inf, as IEEE does)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def recip32(d):
    """RN32(1 / d), and 0 where d == 0."""
    safe = np.where(d == 0, 1.0, d)
    return np.where(d == 0, 0.0, r32(1.0 / safe))


def tile_bytes(fmt):
    if fmt in ASYM:
        return P.asym_tile_bytes(ASYM[fmt])
    return P.tile_bytes(4 if fmt == FP4 else fmt)


# -- encode ------------------------------------------------------------------

def _encode_sym(bits, x):
    Q = 1 << (bits - 1)
    xb = x.reshape(-1, 32)
    m = np.abs(xb).max(axis=1)
    d_bits = P.f16_bits(np.minimum(m / Q, 65504.0))   # m / Q is exact
    e = recip32(P.f16_value(d_bits))
    with np.errstate(invalid="ignore"):
        v = r32(xb * e[:, None])
    codes = np.rint(np.clip(v, -Q, Q - 1)).astype(np.int64) + Q
    return P.pack(bits, codes.reshape(-1, 2048), d_bits.reshape(-1, 64))


def _encode_asym(bits, x):
    qm = (1 << bits) - 1
    g = x.reshape(-1, 128)
    lo = np.minimum(g.min(axis=1), 0.0)
    hi = np.maximum(g.max(axis=1), 0.0)
    s_bits = P.f16_bits(np.minimum(r32(r32(hi - lo) / qm), 65504.0))
    e = recip32(P.f16_value(s_bits))
    z = np.clip(np.rint(r32(-lo * e)), 0, qm)
    with np.errstate(invalid="ignore"):
        q = np.clip(np.rint(r32(g * e[:, None])) + z[:, None], 0, qm).astype(np.int64)
    return P.asym_pack(bits, q.reshape(-1, 2048), s_bits.reshape(-1, 16),
                       z.astype(np.int64).reshape(-1, 16))


def _encode_fp4(x):
    xb = x.reshape(-1, 32)
    m = np.abs(xb).max(axis=1)
    d_bits = P.f16_bits(np.minimum(r32(m / 6.0), 65504.0))
    e = recip32(P.f16_value(d_bits))
    with np.errstate(invalid="ignore"):
        v = r32(xb * e[:, None]).ravel()
    codes = P.fp4_nearest(v)
    return P.pack(4, codes.reshape(-1, 2048), d_bits.reshape(-1, 64))


def encode_values(fmt, x):
    """Packed bytes of float64 values x (each exact in the I/O dtype)."""
    x = np.asarray(x, np.float64).ravel()
    assert x.size % 2048 == 0
    if fmt in SYM:
        return _encode_sym(fmt, x)
    if fmt in ASYM:
        return _encode_asym(ASYM[fmt], x)
    assert fmt == FP4
    return _encode_fp4(x)


def encode(fmt, dtype, xbits):
    return encode_values(fmt, P.dtype_value(dtype, xbits))


# -- decode ------------------------------------------------------------------

def decode_f32(fmt, packed, n):
    """Exact decoded values (float64 holding binary32 values)."""
    packed = np.asarray(packed, np.uint8)[: n // 2048 * tile_bytes(fmt)]
    if fmt in ASYM:
        codes, sb, zp = P.asym_unpack(ASYM[fmt], packed)
        s = P.f16_value(sb)
        y = (codes.reshape(-1, 16, 128) - zp[:, :, None]) * s[:, :, None]
        return y.ravel()
    bits = 4 if fmt == FP4 else fmt
    codes, sb = P.unpack(bits, packed)
    d = P.f16_value(sb)[:, :, None]
    c = codes.reshape(-1, 64, 32)
    if fmt == FP4:
        mag = P.FP4_MAG[c & 7]
        val = np.where(c & 8, -mag, mag)
    else:
        val = c - (1 << (bits - 1))
    return (val * d).ravel()


def decode(fmt, dtype, packed, n):
    return P.dtype_bits(dtype, decode_f32(fmt, packed, n))


# -- reduce ------------------------------------------------------------------

def reduce_mixed(fmt_in, fmt_out, dtype, ranks, n):
    """(packed_out, y bits) of the compressed-domain reduction."""
    s = decode_f32(fmt_in, ranks[0], n)
    for r in ranks[1:]:
        with np.errstate(invalid="ignore"):
            s = r32(s + decode_f32(fmt_in, r, n))
    z = P.dtype_value(dtype, P.dtype_bits(dtype, s))
    out = encode_values(fmt_out, z)
    return out, decode(fmt_out, dtype, out, n)
