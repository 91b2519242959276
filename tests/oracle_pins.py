"""Pins of the CPU oracle to what the pages and the mathematics fix.

Every ``pin_*`` function takes an ``oracle.Oracle`` and raises ``AssertionError``
when the oracle disagrees.  None of them re-derives an expected value by
calling the oracle on the same question: expected values come from the pages
(golden fixtures under ``tests/golden/``, each with its citation), from closed
forms built into the inputs (power-of-two scales, exact multiples of a scale),
from invariants (error bounds, extreme values), or from independent library
routines (numpy / torch IEEE conversions, float64 reciprocals).

The same functions are run against deliberately broken builds of the oracle
(``test_oracle_mutants.py``) to show that a plausible mistake fails at least
one of them.
"""
import os
import re

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TILE = 2048
BLOCK = 32
BITS = (3, 4, 8)
DTYPES = ("fp16", "bf16")


# ---------------------------------------------------------------------------
# independent helpers (layout rule and IEEE conversions, not the oracle's code)
# ---------------------------------------------------------------------------

def qmax(bits):
    return 1 << (bits - 1)


def tile_bytes(bits):
    return TILE * bits // 8 + 2 * (TILE // BLOCK)


def scale_offset(bits):
    return TILE * bits // 8


def unpack(bits, packed):
    """Codes (T, 2048) and raw fp16 scale bits (T, 64) from packed tiles."""
    t = np.asarray(packed, np.uint8).reshape(-1, tile_bytes(bits))
    so = scale_offset(bits)
    scales = t[:, so:so + 128].copy().view("<u2")
    if bits == 8:
        codes = t[:, :2048].astype(np.int64)
    elif bits == 4:
        words = t[:, :1024].copy().view("<u4").astype(np.int64)          # (T, 256)
        codes = (words[:, :, None] >> (4 * np.arange(8))) & 15          # (T, 256, 8)
        codes = codes.reshape(-1, 2048)
    else:
        q2 = t[:, :512].copy().view("<u2").astype(np.int64)             # (T, 256)
        q1 = t[:, 512:768].astype(np.int64)                             # (T, 256)
        low = (q2[:, :, None] >> (2 * np.arange(8))) & 3
        high = (q1[:, :, None] >> np.arange(8)) & 1
        codes = (low | (high << 2)).reshape(-1, 2048)
    return codes, scales


def pack(bits, codes, scale_bits):
    """Packed tiles from codes (T, 2048) and fp16 scale bits (T, 64), by the layout rule."""
    codes = np.asarray(codes, np.int64).reshape(-1, 2048)
    T = codes.shape[0]
    out = np.zeros((T, tile_bytes(bits)), np.uint8)
    if bits == 8:
        out[:, :2048] = codes
    elif bits == 4:
        c = codes.reshape(T, 256, 8)
        words = np.zeros((T, 256), np.uint32)
        for j in range(8):
            words |= (c[:, :, j] << (4 * j)).astype(np.uint32)
        out[:, :1024] = words.view(np.uint8).reshape(T, 1024)
    else:
        c = codes.reshape(T, 256, 8)
        q2 = np.zeros((T, 256), np.uint16)
        q1 = np.zeros((T, 256), np.uint8)
        for j in range(8):
            q2 |= ((c[:, :, j] & 3) << (2 * j)).astype(np.uint16)
            q1 |= (((c[:, :, j] >> 2) & 1) << j).astype(np.uint8)
        out[:, :512] = q2.view(np.uint8).reshape(T, 512)
        out[:, 512:768] = q1
    so = scale_offset(bits)
    out[:, so:so + 128] = np.asarray(scale_bits, np.uint16).reshape(T, 64).view(np.uint8).reshape(T, 128)
    return out.ravel()


def f16_bits(x):
    """IEEE round-to-nearest-even to binary16; overflow to +-inf is the IEEE result."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def f16_value(b):
    return np.asarray(b, np.uint16).view(np.float16).astype(np.float64)


def bf16_value(b):
    """Value of bfloat16 bit patterns (NaN patterns give NaN)."""
    with np.errstate(invalid="ignore"):
        return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits(x):
    """Nearest bfloat16 (ties to even) of float64 values, via torch's conversion."""
    import torch
    t = torch.from_numpy(np.asarray(x, np.float64).astype(np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dtype_bits(dtype, x):
    """dtype bit patterns of float64 values that are exact in binary32."""
    x = np.asarray(x, np.float64)
    assert np.all(x.astype(np.float32).astype(np.float64) == x)
    return f16_bits(x) if dtype == "fp16" else bf16_bits(x)


def dtype_value(dtype, b):
    return f16_value(b) if dtype == "fp16" else bf16_value(b)


def pow2_f16_bits(k):
    """fp16 bits of 2^k built from the format fields (normal or subnormal)."""
    if k >= -14:
        return (k + 15) << 10
    return 1 << (k + 24)


def all_finite(dtype):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = dtype_value(dtype, b)
    keep = np.isfinite(v)
    return b[keep], v[keep]


def pad_tiles(blocks):
    """Stack (nb, 32) blocks into whole tiles (nb rounded up to 64 blocks with zeros)."""
    nb = blocks.shape[0]
    nt = -(-nb // 64)
    out = np.zeros((nt * 64, BLOCK), blocks.dtype)
    out[:nb] = blocks
    return out.reshape(-1)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------------------
# P1: tile byte counts printed on the page
# ---------------------------------------------------------------------------

def pin_tile_bytes(o):
    for fmt, n, nbytes in read_golden("tile_bytes.txt"):
        bits = {"INT4": 4, "INT3": 3}[fmt]
        assert o.packed_bytes(bits, int(n)) == int(nbytes), (fmt, o.packed_bytes(bits, int(n)))
        for t in (1, 3, 64):
            assert o.packed_bytes(bits, t * int(n)) == t * int(nbytes)
    # INT8 extends the same framework (2048 B of codes + 128 B of scales).
    assert o.packed_bytes(8, 2048) == 2176
    for bits in BITS:
        assert o.packed_bytes(bits, 2047) == 0 and o.packed_bytes(bits, 2048 + 32) == 0
    # and the buffer the oracle writes has exactly that size
    for bits in BITS:
        p = o.encode(bits, "fp16", np.zeros(4096, np.uint16))
        assert p.size == 2 * tile_bytes(bits)


# ---------------------------------------------------------------------------
# P6: bit order inside a unit and scale placement
# ---------------------------------------------------------------------------

def _block_with_codes(bits, codes8, s=1.0):
    """32 values whose block quantizes to `codes8` in unit 0 (scale s exactly).

    Unit 1 holds the anchor -Q*s (code 0) so the block maximum is Q*s."""
    Q = qmax(bits)
    k = np.zeros(BLOCK, np.float64)
    k[:8] = np.asarray(codes8, np.float64) - Q
    k[8] = -Q
    return k * s


def pin_unit_bit_order(o):
    for row in read_golden("unit_bit_order.txt"):
        fmt, codes = row[0], [int(c) for c in row[1].split(",")]
        expect = dict(kv.split("=") for kv in row[2:])
        bits = {"INT4": 4, "INT3": 3}[fmt]
        for dtype in DTYPES:
            x = np.zeros(TILE, np.float64)
            x[:BLOCK] = _block_with_codes(bits, codes)
            p = o.encode(bits, dtype, dtype_bits(dtype, x))
            if bits == 4:
                word = int(p[0:4].view("<u4")[0])
                assert word == int(expect["word"], 16), (dtype, codes, hex(word))
            else:
                q2 = int(p[0:2].view("<u2")[0])
                q1 = int(p[512])
                assert q2 == int(expect["q2"], 16), (dtype, codes, hex(q2))
                assert q1 == int(expect["q1"], 16), (dtype, codes, hex(q1))


def pin_scale_placement(o):
    """Block g's scale sits at scale_offset + 2g, little-endian fp16."""
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            x = np.zeros((2 * 64, BLOCK), np.float64)
            exps = np.array([(g * 7) % 21 - 12 for g in range(128)])
            for g in range(128):
                s = 2.0 ** exps[g]
                x[g, g % BLOCK] = -Q * s           # anchor at a varying position
                x[g, (g + 5) % BLOCK] = (Q - 1) * s
            p = o.encode(bits, dtype, dtype_bits(dtype, x.ravel()))
            codes, scales = unpack(bits, p)
            want = np.array([pow2_f16_bits(int(e)) for e in exps], np.uint16).reshape(2, 64)
            assert np.array_equal(scales, want), (bits, dtype)
            c = codes.reshape(128, BLOCK)
            for g in range(128):
                assert c[g, g % BLOCK] == 0 and c[g, (g + 5) % BLOCK] == 2 * Q - 1
            # every other position in each block decodes to zero -> code Q
            mask = np.ones((128, BLOCK), bool)
            mask[np.arange(128), np.arange(128) % BLOCK] = False
            mask[np.arange(128), (np.arange(128) + 5) % BLOCK] = False
            assert np.all(c[mask] == Q)


# ---------------------------------------------------------------------------
# P3: exact round trip of multiples k*s of a representable scale
# ---------------------------------------------------------------------------

def _exact_scales(bits, dtype):
    """Scales s (fp16 values) such that every k*s, |k| <= Q, is exact in dtype."""
    Q = qmax(bits)
    sig = 11 if dtype == "fp16" else 8
    kbits = max(1, (Q - 1).bit_length())   # |k| <= Q-1 needs this many bits; Q itself is a power of 2
    out = []
    for m in (1, 3, 5, 7):
        if m.bit_length() + kbits > sig:
            continue
        for e in (-20, -12, -5, 0, 3):
            s = m * 2.0 ** e
            if Q * s > 60000 or s < 2.0 ** -14:
                continue
            out.append(s)
    return out


def pin_exact_roundtrip(o, seed=1):
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            scales = _exact_scales(bits, dtype)
            nb = 64 * 3
            k = rng.integers(-Q, Q, size=(nb, BLOCK))
            k[np.arange(nb), rng.integers(0, BLOCK, nb)] = -Q          # anchor
            s = np.array([scales[i % len(scales)] for i in range(nb)])
            x = (k * s[:, None]).ravel()
            xb = dtype_bits(dtype, x)
            p = o.encode(bits, dtype, xb)
            codes, sb = unpack(bits, p)
            assert np.array_equal(codes.reshape(nb, BLOCK), k + Q), (bits, dtype)
            assert np.array_equal(sb.ravel(), f16_bits(s)), (bits, dtype)
            y = o.decode(bits, dtype, p, x.size)
            assert np.array_equal(y, xb), (bits, dtype)
            yf = o.decode_f32(bits, p, x.size)
            assert np.array_equal(yf.astype(np.float64), x), (bits, dtype)


# ---------------------------------------------------------------------------
# P2: extreme values land on the ends of the code range
# ---------------------------------------------------------------------------

def pin_extremes_and_grid(o, seed=2):
    """The block's largest |x| maps to code 0 (negative) or 2Q-1 (positive), and
    every decoded value is an integer in [-Q, Q-1] times the block scale."""
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            nb = 64 * 4
            x = rng.standard_normal((nb, BLOCK)) * np.exp(rng.uniform(-3, 6, size=(nb, 1)))
            xb = dtype_bits(dtype, x.astype(np.float32).astype(np.float64)) if dtype == "bf16" else \
                f16_bits(x)
            xv = dtype_value(dtype, xb).reshape(nb, BLOCK)
            p = o.encode(bits, dtype, xb)
            codes, sb = unpack(bits, p)
            codes = codes.reshape(nb, BLOCK)
            d = f16_value(sb.ravel())
            # only blocks whose scale is a normal fp16 value (full relative precision)
            ok = d >= 2.0 ** -14
            assert ok.mean() > 0.9
            i = np.argmax(np.abs(xv), axis=1)
            ext = codes[np.arange(nb), i]
            neg = xv[np.arange(nb), i] < 0
            assert np.all(ext[neg & ok] == 0) and np.all(ext[~neg & ok] == 2 * Q - 1), (bits, dtype)
            assert np.all((codes >= 0) & (codes <= 2 * Q - 1))
            y = o.decode_f32(bits, p, nb * BLOCK).astype(np.float64).reshape(nb, BLOCK)
            kk = y[ok] / d[ok, None]
            assert np.array_equal(kk, (codes - Q)[ok]), (bits, dtype)


# ---------------------------------------------------------------------------
# P4: zero, tiny and huge blocks
# ---------------------------------------------------------------------------

def pin_zero_tiny_huge(o):
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            # all +0 / -0
            xb = np.zeros(TILE, np.uint16)
            xb[1::2] = 0x8000
            p = o.encode(bits, dtype, xb)
            codes, sb = unpack(bits, p)
            assert np.all(codes == Q) and np.all(sb == 0)
            assert np.all(o.decode(bits, dtype, p, TILE) == 0)       # +0 everywhere
        # bf16 blocks whose m/Q is below half the smallest fp16 subnormal flush to 0
        tiny = np.zeros(TILE, np.float64)
        tiny[:BLOCK] = 2.0 ** -130 * np.sign(np.arange(BLOCK) - 15.5)
        tiny[BLOCK] = Q * 2.0 ** -25                              # m/Q = 2^-25: tie -> 0
        tiny[2 * BLOCK] = Q * 2.0 ** -25 * (1 + 2.0 ** -7)        # just above: -> 2^-24
        tiny[2 * BLOCK + 1] = -Q * 2.0 ** -25 * (1 + 2.0 ** -7)
        p = o.encode(bits, "bf16", dtype_bits("bf16", tiny))
        codes, sb = unpack(bits, p)
        assert sb[0, 0] == 0 and sb[0, 1] == 0 and sb[0, 2] == 0x0001, sb[0, :3]
        assert np.all(codes[0, :2 * BLOCK] == Q)
        # scale 2^-24, multiplier 2^24: the values scale to +-(Q/2)(1 + 2^-7)
        half = np.rint(Q / 2 * (1 + 2.0 ** -7))
        assert codes[0, 2 * BLOCK] == Q + half and codes[0, 2 * BLOCK + 1] == Q - half
        # bf16 block far above 65504*Q saturates the scale at 65504
        huge = np.zeros(TILE, np.float64)
        huge[:4] = [2.0 ** 24, -2.0 ** 24, 65504.0, -65504.0]
        p = o.encode(bits, "bf16", dtype_bits("bf16", huge))
        codes, sb = unpack(bits, p)
        assert sb[0, 0] == 0x7BFF
        assert codes[0, 0] == 2 * Q - 1 and codes[0, 1] == 0
        assert codes[0, 2] == Q + 1 and codes[0, 3] == Q - 1


# ---------------------------------------------------------------------------
# P5: brute force over tiny blocks with a power-of-two scale
# ---------------------------------------------------------------------------

def _pow2_exponents(bits):
    Q = qmax(bits)
    top = 15 - (bits - 1)          # Q * 2^k must stay a finite fp16 value
    return [-24, -20, -14, -9, -1, 0, 3, top]


def pin_bruteforce_pow2(o, stride=1):
    """Every finite dtype value x with |x| <= Q*2^k in the block [-Q*2^k, x, 0...]:
    the scale is 2^k, the multiplier 2^-k, so the code is the closed form
    clip(round_half_even(x / 2^k), -Q, Q-1) + Q, evaluated exactly in float64."""
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            allb, allv = all_finite(dtype)
            for k in _pow2_exponents(bits):
                a = Q * 2.0 ** k
                sel = np.abs(allv) <= a
                xb, xv = allb[sel][::stride], allv[sel][::stride]
                nb = xb.size
                blocks = np.zeros((nb, BLOCK), np.uint16)
                blocks[:, 0] = dtype_bits(dtype, np.array([-a]))[0]
                blocks[:, 1] = xb
                p = o.encode(bits, dtype, pad_tiles(blocks))
                codes, sb = unpack(bits, p)
                codes = codes.reshape(-1, BLOCK)[:nb]
                want = np.clip(np.rint(xv / 2.0 ** k), -Q, Q - 1) + Q
                bad = codes[:, 1] != want
                assert not bad.any(), (bits, dtype, k, xv[bad][:4], codes[bad, 1][:4], want[bad][:4])
                assert np.all(codes[:, 0] == 0)
                assert np.all(sb.ravel()[:nb] == pow2_f16_bits(k))


def pin_bruteforce_general_scale(o):
    """Blocks [-Q*d, x, 0...] with d a non-power-of-two fp16 value and every
    finite fp16 x with |x| <= Q*d.  The scale is d exactly and the encode
    multiplier e = RN32(1/d) (the reading that the page's encode scale is a
    multiplier kept in fp32).  The code is clip(round_half_even(RN32(x*e))) + Q,
    with x*e formed exactly in float64 and rounded once to float32.  Some x lie
    where x*e and x/d round to different codes (for scales such as 0x0F90,
    0x17A8, 0x3368), so the check also separates "multiply by e" from "divide by d"."""
    allb, allv = all_finite("fp16")
    for bits in BITS:
        Q = qmax(bits)
        diff_seen = 0
        for d_bits in (0x3555, 0x2E66, 0x3BFF, 0x0F90, 0x17A8, 0x3368, 0x0123):
            d = float(f16_value(np.uint16(d_bits)))
            a = Q * d
            if f16_value(f16_bits(a)) != a:
                continue
            sel = np.abs(allv) <= a
            xb, xv = allb[sel], allv[sel]
            nb = xb.size
            blocks = np.zeros((nb, BLOCK), np.uint16)
            blocks[:, 0] = f16_bits(-a)
            blocks[:, 1] = xb
            p = o.encode(bits, "fp16", pad_tiles(blocks))
            codes, sb = unpack(bits, p)
            codes = codes.reshape(-1, BLOCK)[:nb]
            assert np.all(sb.ravel()[:nb] == d_bits)
            e = np.float64(np.float32(1.0 / d))
            v = (xv * e).astype(np.float32).astype(np.float64)
            want = np.clip(np.rint(v), -Q, Q - 1) + Q
            bad = codes[:, 1] != want
            assert not bad.any(), (bits, hex(d_bits), xv[bad][:4], codes[bad, 1][:4], want[bad][:4])
            by_div = np.clip(np.rint((xv / d).astype(np.float32).astype(np.float64)), -Q, Q - 1) + Q
            diff_seen += int((by_div != want).sum())
        assert diff_seen > 0, bits


def pin_scale_reciprocal_exhaustive(o):
    """For every positive finite fp16 d: a block maximum of Q*d gives scale d and
    multiplier RN32(1/d), taken from a float64 division rounded once to float32
    (double rounding is harmless here: 53 >= 2*24 + 2)."""
    d_bits = np.arange(1, 0x7C00, dtype=np.uint16)
    d = f16_value(d_bits)
    for bits in BITS:
        Q = qmax(bits)
        for i in range(0, d_bits.size, 1):
            db, e = o.block_scale(bits, float(np.float32(Q * d[i])))
            if db != d_bits[i] or e != np.float32(1.0 / d[i]):
                raise AssertionError((bits, hex(int(d_bits[i])), hex(db), e, np.float32(1.0 / d[i])))
        assert o.block_scale(bits, 0.0) == (0, 0.0)
        db, e = o.block_scale(bits, 65504.0 * Q * 4)
        assert db == 0x7BFF and e == np.float32(1.0 / 65504.0)
        # arbitrary maxima: scale = nearest fp16 of m/Q (numpy's correctly rounded conversion)
        rng = np.random.default_rng(bits)
        ms = (rng.standard_normal(2000) * np.exp(rng.uniform(-20, 12, 2000))).astype(np.float32)
        for m in np.abs(ms):
            db, _ = o.block_scale(bits, float(m))
            want = f16_bits(np.float64(m) / Q)
            if float(m) / Q > 65504:
                want = np.uint16(0x7BFF)
            assert db == want, (bits, m, hex(db), hex(int(want)))


# ---------------------------------------------------------------------------
# IEEE conversions against numpy / torch
# ---------------------------------------------------------------------------

def _f32_probe_values(seed=3):
    rng = np.random.default_rng(seed)
    bitsr = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    rnd = bitsr.view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    # values near every fp16 value and every midpoint between neighbours
    b16, v16 = all_finite("fp16")
    v16 = np.sort(np.unique(v16))
    mids = (v16[:-1] + v16[1:]) / 2                       # exact in float64; exact in f32 too
    near = np.concatenate([v16, mids]).astype(np.float32)
    up = np.nextafter(near, np.float32(np.inf))
    dn = np.nextafter(near, np.float32(-np.inf))
    special = np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e30, 2.0 ** -25, 2.0 ** -24,
                        2.0 ** -25 * 1.5, 2.0 ** -14, 2.0 ** -149, 3.4e38], np.float32)
    return np.concatenate([rnd, near, up, dn, special, -special])


def pin_f16_conversions(o):
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.f16_to_f32(b)
    want = b.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    x = _f32_probe_values()
    got = o.f32_to_f16(x)
    with np.errstate(over="ignore"):   # values beyond the binary16 range round to +-inf
        want = x.astype(np.float16).view(np.uint16)
    bad = got != want
    assert not bad.any(), (x[bad][:5], got[bad][:5], want[bad][:5])


def pin_bf16_conversions(o):
    import torch
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = o.bf16_to_f32(b)
    want = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
    x = _f32_probe_values(4)
    xb = np.concatenate([x, (x.view(np.uint32) & 0xFFFF0000 | 0x8000).view(np.float32)])  # bf16 ties
    xb = xb[np.isfinite(xb)]
    got = o.f32_to_bf16(xb)
    want = torch.from_numpy(xb).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = got != want
    assert not bad.any(), (xb[bad][:5], got[bad][:5], want[bad][:5])


# ---------------------------------------------------------------------------
# decode rounding to the I/O dtype
# ---------------------------------------------------------------------------

def pin_decode_rounding(o, seed=5):
    """decode = dtype_RNE((code - Q) * scale) for arbitrary codes and scales,
    the product evaluated exactly in float64, the rounding by numpy / torch."""
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        T = 4
        codes = rng.integers(0, 2 * Q, size=(T, 2048))
        sbits = rng.integers(0, 0x7C00, size=(T, 64)).astype(np.uint16)
        p = pack(bits, codes, sbits)
        exact = (codes - Q).reshape(T, 64, BLOCK) * f16_value(sbits)[:, :, None]
        exact = exact.ravel()
        yf = o.decode_f32(bits, p, T * 2048).astype(np.float64)
        assert np.array_equal(yf, exact), bits
        for dtype in DTYPES:
            y = o.decode(bits, dtype, p, T * 2048)
            want = f16_bits(exact) if dtype == "fp16" else bf16_bits(exact)
            assert np.array_equal(y, want), (bits, dtype)


# ---------------------------------------------------------------------------
# P7: reduction special cases
# ---------------------------------------------------------------------------

def _rng_blocks(rng, dtype, nb, scale_lo=-4, scale_hi=4):
    x = rng.standard_normal((nb, BLOCK)) * np.exp(rng.uniform(scale_lo, scale_hi, size=(nb, 1)))
    x[rng.random((nb, BLOCK)) < 0.01] *= 50
    return dtype_bits(dtype, x.astype(np.float32).astype(np.float64)).ravel() if dtype == "bf16" \
        else f16_bits(x).ravel()


def pin_reduce_r1_composition(o, seed=6):
    """R = 1: the reduction re-quantizes dtype_RNE(exact decode) and decodes it.
    The packed result equals encoding the decoded-and-rounded values (rounding by
    numpy / torch); the output equals dtype_RNE((code-Q)*scale) of that result."""
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            n = 2 * TILE
            xb = _rng_blocks(rng, dtype, n // BLOCK)
            p = o.encode(bits, dtype, xb)
            codes, sb = unpack(bits, p)
            exact = ((codes - Q).reshape(-1, 64, BLOCK) * f16_value(sb)[:, :, None]).ravel()
            zb = f16_bits(exact) if dtype == "fp16" else bf16_bits(exact)
            want_packed = o.encode(bits, dtype, zb)
            out, y = o.reduce(bits, dtype, [p], n)
            assert np.array_equal(out, want_packed), (bits, dtype)
            c2, s2 = unpack(bits, out)
            ex2 = ((c2 - Q).reshape(-1, 64, BLOCK) * f16_value(s2)[:, :, None]).ravel()
            want_y = f16_bits(ex2) if dtype == "fp16" else bf16_bits(ex2)
            assert np.array_equal(y, want_y), (bits, dtype)


def pin_reduce_exact_common_scale(o, seed=7):
    """All ranks of a block share a scale s; every element's integer sum stays in
    [-Q, Q-1] and one element sums to -Q.  Then every partial sum is exact, the
    summed block has scale s again, and the output equals the exact sum."""
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        for dtype in DTYPES:
            scales = _exact_scales(bits, dtype)
            for R in (1, 2, 3, 4, 8):
                nb = 128
                k = np.zeros((R, nb, BLOCK), np.int64)
                for b in range(nb):
                    for r in range(R):
                        k[r, b, r] = -Q                       # rank r's anchor at element r
                        k[(r + 1) % R, b, r] += Q - 1 if R > 1 else 0   # keeps element r's sum at -1 (R>1)
                    # element R sums to exactly -Q
                    if R == 1:
                        k[0, b, R] = -Q
                    else:
                        k[0, b, R] = -(Q // 2)
                        k[1, b, R] = -(Q // 2)
                    # the rest: random sums in [-Q, Q-1] split over the ranks
                    for e in range(R + 1, BLOCK):
                        tot = int(rng.integers(-Q, Q))
                        parts = np.zeros(R, np.int64)
                        left = tot
                        for r in range(R - 1):
                            lo, hi = max(-Q, left - (Q - 1) * (R - 1 - r)), min(Q - 1, left + Q * (R - 1 - r))
                            parts[r] = int(rng.integers(lo, hi + 1))
                            left -= parts[r]
                        parts[R - 1] = left
                        k[:, b, e] = parts
                assert np.all((k >= -Q) & (k <= Q - 1))
                tot = k.sum(axis=0)
                assert np.all((tot >= -Q) & (tot <= Q - 1)) and np.all((tot == -Q).any(axis=1))
                s = np.array([scales[i % len(scales)] for i in range(nb)])
                ranks = [o.encode(bits, dtype, dtype_bits(dtype, (k[r] * s[:, None]).ravel()))
                         for r in range(R)]
                out, y = o.reduce(bits, dtype, ranks, nb * BLOCK)
                codes, sb = unpack(bits, out)
                assert np.array_equal(codes.reshape(nb, BLOCK), tot + Q), (bits, dtype, R)
                assert np.array_equal(sb.ravel(), f16_bits(s)), (bits, dtype, R)
                assert np.array_equal(y, dtype_bits(dtype, (tot * s[:, None]).ravel())), (bits, dtype, R)


def _golden_expect(name):
    rows = read_golden(name)
    scale = int(rows[0][1], 16)
    elems = {r[0]: (int(r[1]), int(r[2], 16)) for r in rows[1:]}
    return scale, elems


def pin_reduce_rank_order(o):
    scale, elems = _golden_expect("reduce_rank_order.txt")
    A, B, E2, E3 = 0, 1, 2, 3
    vals = np.zeros((4, TILE), np.float64)
    vals[0, [A, E2, E3]] = [-16, 2, 14]
    vals[1, [A, B]] = [-2.0 ** -20, -2.0 ** -17]
    vals[2, [A, E2, E3]] = [14, -16, 2]
    vals[3, [A, E2, E3]] = [2, 14, -16]
    ranks = [o.encode(4, "fp16", f16_bits(v)) for v in vals]
    out, y = o.reduce(4, "fp16", ranks, TILE)
    codes, sb = unpack(4, out)
    assert sb[0, 0] == scale, hex(sb[0, 0])
    for name, idx in (("A", A), ("B", B), ("E2", E2), ("E3", E3)):
        code, ybits = elems[name]
        assert codes[0, idx] == code, (name, codes[0, idx])
        assert y[idx] == ybits, (name, hex(y[idx]))
    assert np.all(codes[0, 4:BLOCK] == 8)


def pin_reduce_exact_terms(o):
    scale, elems = _golden_expect("reduce_exact_terms.txt")
    c0 = np.full((1, 2048), 128)
    c1 = np.full((1, 2048), 128)
    s0 = np.zeros((1, 64), np.uint16)
    s1 = np.zeros((1, 64), np.uint16)
    c0[0, 0], s0[0, 0] = 255, 0x3FFF
    c1[0, 0], s1[0, 0] = 2, 0x4004
    ranks = [pack(8, c0, s0), pack(8, c1, s1)]
    out, y = o.reduce(8, "fp16", ranks, TILE)
    codes, sb = unpack(8, out)
    assert sb[0, 0] == scale, hex(sb[0, 0])
    code, ybits = elems["0"]
    assert codes[0, 0] == code and y[0] == ybits, (codes[0, 0], hex(y[0]))
    assert np.all(codes[0, 1:] == 128) and np.all(y[1:] == 0)


# ---------------------------------------------------------------------------
# mixed formats per phase (inputs in one format, re-encoded sum in another)
# ---------------------------------------------------------------------------

MIXED = [(4, 8), (3, 4), (3, 8), (8, 4), (4, 3)]


def pin_reduce_mixed_r1_composition(o, seed=9):
    """R = 1 with input format a and output format b: the packed result is the
    encoding in b of dtype_RNE(exact decode of a) (rounding by numpy / torch),
    and the output is dtype_RNE of its exact decode in b."""
    rng = np.random.default_rng(seed)
    for a, b in MIXED:
        Qb = qmax(b)
        for dtype in DTYPES:
            n = 2 * TILE
            xb = _rng_blocks(rng, dtype, n // BLOCK)
            p = o.encode(a, dtype, xb)
            codes, sb = unpack(a, p)
            exact = ((codes - qmax(a)).reshape(-1, 64, BLOCK) * f16_value(sb)[:, :, None]).ravel()
            zb = f16_bits(exact) if dtype == "fp16" else bf16_bits(exact)
            out, y = o.reduce_mixed(a, b, dtype, [p], n)
            assert out.size == sym_packed_bytes(b, n)
            assert np.array_equal(out, o.encode(b, dtype, zb)), (a, b, dtype)
            c2, s2 = unpack(b, out)
            ex2 = ((c2 - Qb).reshape(-1, 64, BLOCK) * f16_value(s2)[:, :, None]).ravel()
            assert np.array_equal(y, f16_bits(ex2) if dtype == "fp16" else bf16_bits(ex2)), (a, b, dtype)


def sym_packed_bytes(bits, n):
    return n // TILE * tile_bytes(bits)


def pin_reduce_mixed_exact(o, seed=10):
    """INT4 inputs sharing a power-of-two scale s over R = 8 ranks, integer sums
    in [-64, 63] with one element at -64: the INT8 re-encode has scale s/2 and
    codes 2*sum + 128, and the output equals the exact sum.  Likewise INT3
    inputs over R = 2 (sums in [-8, 6], one at -8) re-encoded in INT4 with
    scale s and codes sum + 8."""
    rng = np.random.default_rng(seed)
    for a, b, R, lo, hi in ((4, 8, 8, -64, 63), (3, 4, 2, -8, 6)):
        Qa = qmax(a)
        for dtype in DTYPES:
            nb = 128
            k = rng.integers(-Qa, Qa, size=(R, nb, BLOCK))
            k[:, :, 0] = -Qa                    # every rank's anchor; element 0 sums to -R*Qa
            tot = k.sum(axis=0)
            assert tot[:, 0].min() == lo
            k = np.where((tot > hi)[None], 0, k)
            k[:, :, 0] = -Qa
            tot = k.sum(axis=0)
            assert np.all((tot >= lo) & (tot <= hi))
            s = 2.0 ** rng.integers(-8, 3, size=nb)
            ranks = [o.encode(a, dtype, dtype_bits(dtype, (k[r] * s[:, None]).ravel())) for r in range(R)]
            out, y = o.reduce_mixed(a, b, dtype, ranks, nb * BLOCK)
            codes, sb = unpack(b, out)
            scale = s * (-lo) / qmax(b)          # 2^-1 * s for (4, 8), s for (3, 4)
            assert np.array_equal(sb.ravel(), f16_bits(scale)), (a, b, dtype)
            assert np.array_equal(codes.reshape(nb, BLOCK), (tot / (scale / s)[:, None]).astype(np.int64) + qmax(b))
            assert np.array_equal(y, dtype_bits(dtype, (tot * s[:, None]).ravel())), (a, b, dtype)


# ---------------------------------------------------------------------------
# asymmetric group-128 codec (scale + zero point per 128 values)
# ---------------------------------------------------------------------------

ASYM = {4: 20, 8: 24}   # bits -> format id
AGROUP = 128


def asym_tile_bytes(bits):
    return TILE * bits // 8 + 3 * (TILE // AGROUP)


def asym_unpack(bits, packed):
    """Codes (T, 2048), scale bits (T, 16), zero points (T, 16) of asymmetric tiles."""
    t = np.asarray(packed, np.uint8).reshape(-1, asym_tile_bytes(bits))
    cb = TILE * bits // 8
    if bits == 8:
        codes = t[:, :2048].astype(np.int64)
    else:
        words = t[:, :1024].copy().view("<u4").astype(np.int64)
        codes = ((words[:, :, None] >> (4 * np.arange(8))) & 15).reshape(-1, 2048)
    scales = t[:, cb:cb + 32].copy().view("<u2")
    zeros = t[:, cb + 32:cb + 48].astype(np.int64)
    return codes, scales, zeros


def asym_pack(bits, codes, scale_bits, zeros):
    codes = np.asarray(codes, np.int64).reshape(-1, 2048)
    T = codes.shape[0]
    out = np.zeros((T, asym_tile_bytes(bits)), np.uint8)
    cb = TILE * bits // 8
    if bits == 8:
        out[:, :2048] = codes
    else:
        c = codes.reshape(T, 256, 8)
        words = np.zeros((T, 256), np.uint32)
        for j in range(8):
            words |= (c[:, :, j] << (4 * j)).astype(np.uint32)
        out[:, :1024] = words.view(np.uint8).reshape(T, 1024)
    out[:, cb:cb + 32] = np.asarray(scale_bits, np.uint16).reshape(T, 16).view(np.uint8).reshape(T, 32)
    out[:, cb + 32:cb + 48] = np.asarray(zeros, np.uint8).reshape(T, 16)
    return out.ravel()


def pin_asym_tile_layout(o):
    for bits, fid in ASYM.items():
        assert o.packed_bytes(fid, 2048) == asym_tile_bytes(bits) == (1072 if bits == 4 else 2096)
        assert o.packed_bytes(fid, 2048 * 5) == 5 * asym_tile_bytes(bits)
        assert o.packed_bytes(fid, 100) == 0
        # codes in the symmetric layout, group scale / zero point at their slots
        x = np.zeros(TILE)
        x[:8] = np.arange(8) - 3.0          # group 0: range [-3, 4]
        x[AGROUP * 5] = 6.0                 # group 5: range [0, 6]
        p = o.encode(fid, "fp16", f16_bits(x))
        codes, sb, zp = asym_unpack(bits, p)
        qmax = (1 << bits) - 1
        assert f16_value(sb[0, 0]) == np.float16(7.0 / qmax) and zp[0, 5] == 0
        assert f16_value(sb[0, 5]) == np.float16(6.0 / qmax)
        assert np.all(sb[0, [1, 2, 3, 4] + list(range(6, 16))] == 0) and np.all(zp[0, 1:] == 0)


def _asym_exact_groups(rng, bits, dtype, ng):
    """Groups of values (k - z) * s with k in [0, qmax], both ends present."""
    qmax = (1 << bits) - 1
    sig = 11 if dtype == "fp16" else 8
    kk = rng.integers(0, qmax + 1, size=(ng, AGROUP))
    kk[:, 0] = 0
    kk[:, 1] = qmax
    z = rng.integers(0, qmax + 1, size=ng)
    s = []
    for g in range(ng):
        m = 3 if (bits == 4 and sig == 11 and g % 2) else 1
        s.append(m * 2.0 ** int(rng.integers(-12, 3)))
    s = np.array(s)
    x = (kk - z[:, None]) * s[:, None]
    return kk, z, s, x


def pin_asym_exact_roundtrip(o, seed=21):
    rng = np.random.default_rng(seed)
    for bits, fid in ASYM.items():
        for dtype in DTYPES:
            ng = 16 * 6
            kk, z, s, x = _asym_exact_groups(rng, bits, dtype, ng)
            xb = dtype_bits(dtype, x.ravel())
            p = o.encode(fid, dtype, xb)
            codes, sb, zp = asym_unpack(bits, p)
            assert np.array_equal(codes.reshape(ng, AGROUP), kk), (bits, dtype)
            assert np.array_equal(zp.ravel(), z), (bits, dtype)
            assert np.array_equal(sb.ravel(), f16_bits(s)), (bits, dtype)
            assert np.array_equal(o.decode(fid, dtype, p, x.size), xb), (bits, dtype)


def pin_asym_bruteforce_pow2(o):
    """Groups [-z*2^m, (qmax-z)*2^m, x, 0...]: scale 2^m, zero point z, and the
    code of x is clamp(round_half_even(x / 2^m) + z, 0, qmax) (float64)."""
    allb, allv = all_finite("fp16")
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        for m, z in ((-14, 0), (-6, 3), (0, qmax // 2), (2, qmax), (-20, 1)):
            lo, hi = -z * 2.0 ** m, (qmax - z) * 2.0 ** m
            sel = (allv >= lo) & (allv <= hi)
            xb, xv = allb[sel], allv[sel]
            nb = xb.size
            groups = np.zeros((nb, AGROUP), np.uint16)
            groups[:, 0] = f16_bits(lo)
            groups[:, 1] = f16_bits(hi)
            groups[:, 2] = xb
            ng = -(-nb // 16) * 16
            buf = np.zeros((ng, AGROUP), np.uint16)
            buf[:nb] = groups
            p = o.encode(fid, "fp16", buf.ravel())
            codes, sb, zp = asym_unpack(bits, p)
            codes = codes.reshape(-1, AGROUP)[:nb]
            want = np.clip(np.rint(xv / 2.0 ** m) + z, 0, qmax)
            bad = codes[:, 2] != want
            assert not bad.any(), (bits, m, z, xv[bad][:4], codes[bad, 2][:4], want[bad][:4])
            assert np.all(zp.ravel()[:nb] == z) and np.all(sb.ravel()[:nb] == pow2_f16_bits(m))


def pin_asym_bruteforce_general_scale(o):
    """Groups [-z*d, (qmax-z)*d, x, 0...] with d a non-power-of-two fp16 scale
    (both ends exact in fp16, so the range divided by qmax is d exactly) and
    every finite fp16 x in the range: scale d, zero point z, and the code of x
    is clamp(round_half_even(RN32(x * RN32(1/d))) + z, 0, qmax), the products
    formed in float64 and rounded once.  For the scales 0x0F80 and 0x3300 some
    x round differently under x / d, so the check also tells "multiply by the
    fp32 reciprocal" from "divide by the scale"."""
    allb, allv = all_finite("fp16")
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        diff_seen = 0
        for d_bits in (0x0F80, 0x3300, 0x0F90, 0x3A00):
            d = float(f16_value(np.uint16(d_bits)))
            for z in (0, qmax, (qmax + 1) // 2, 3):
                lo, hi = -z * d, (qmax - z) * d
                if f16_value(f16_bits(lo)) != lo or f16_value(f16_bits(hi)) != hi:
                    continue
                sel = (allv >= lo) & (allv <= hi)
                xb, xv = allb[sel], allv[sel]
                nb = xb.size
                ng = -(-nb // 16) * 16
                buf = np.zeros((ng, AGROUP), np.uint16)
                buf[:nb, 0] = f16_bits(lo)
                buf[:nb, 1] = f16_bits(hi)
                buf[:nb, 2] = xb
                p = o.encode(fid, "fp16", buf.ravel())
                codes, sb, zp = asym_unpack(bits, p)
                codes = codes.reshape(-1, AGROUP)[:nb]
                assert np.all(sb.ravel()[:nb] == d_bits) and np.all(zp.ravel()[:nb] == z), (bits, hex(d_bits), z)
                e = np.float64(np.float32(1.0 / d))
                want = np.clip(np.rint((xv * e).astype(np.float32).astype(np.float64)) + z, 0, qmax)
                bad = codes[:, 2] != want
                assert not bad.any(), (bits, hex(d_bits), z, xv[bad][:4], codes[bad, 2][:4], want[bad][:4])
                by_div = np.clip(np.rint((xv / d).astype(np.float32).astype(np.float64)) + z, 0, qmax)
                diff_seen += int((by_div != want).sum())
        assert diff_seen > 0, bits


def pin_asym_group_params(o):
    """Every positive finite fp16 scale s and a zero point z: a group range
    [-z*s, (qmax-z)*s] gives scale s, multiplier RN32(1/s) (float64 quotient
    rounded once), zero point z."""
    d_bits = np.arange(1, 0x7C00, 7, dtype=np.uint16)
    d = f16_value(d_bits)
    for bits in (4, 8):
        qmax = (1 << bits) - 1
        for i in range(d_bits.size):
            z = (i * 5) % (qmax + 1)
            lo, hi = np.float32(-z * d[i]), np.float32((qmax - z) * d[i])
            if float(hi) - float(lo) != qmax * d[i] or qmax * d[i] > 65504 * qmax:
                continue
            db, e, zz = o.group_params(bits, lo, hi)
            assert db == d_bits[i] and e == np.float32(1.0 / d[i]) and zz == z, (bits, hex(int(d_bits[i])), z)
        assert o.group_params(bits, 0.0, 0.0) == (0, 0.0, 0)
        db, e, zz = o.group_params(bits, -1e30, 1e30)
        assert db == 0x7BFF


def pin_asym_special_groups(o):
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        for dtype in DTYPES:
            x = np.zeros(TILE)
            x[AGROUP:2 * AGROUP] = 0.5                       # positive only: lo = 0 -> z = 0, all codes qmax
            x[2 * AGROUP:3 * AGROUP] = -0.25                 # negative only: hi = 0 -> z = qmax, codes 0
            x[3 * AGROUP:4 * AGROUP:2] = -0.0                # zeros and -0
            p = o.encode(fid, dtype, dtype_bits(dtype, x))
            codes, sb, zp = asym_unpack(bits, p)
            c = codes.reshape(16, AGROUP)
            assert sb[0, 0] == 0 and zp[0, 0] == 0 and np.all(c[0] == 0)
            assert zp[0, 1] == 0 and np.all(c[1] == qmax)
            assert zp[0, 2] == qmax and np.all(c[2] == 0)
            assert sb[0, 3] == 0 and np.all(c[3] == 0)
            y = dtype_value(dtype, o.decode(fid, dtype, p, TILE))
            assert np.all(y[:AGROUP] == 0) and np.all(y[3 * AGROUP:4 * AGROUP] == 0)
            assert np.all(np.abs(y[AGROUP:2 * AGROUP] - 0.5) <= 0.5 / qmax)


def pin_asym_decode_algorithm1(o, seed=22):
    """Decode = dtype_RNE((q - z) * s) for arbitrary codes, scales and zero points."""
    rng = np.random.default_rng(seed)
    for bits, fid in ASYM.items():
        T = 3
        codes = rng.integers(0, 1 << bits, size=(T, 2048))
        sb = rng.integers(0, 0x7C00, size=(T, 16)).astype(np.uint16)
        zp = rng.integers(0, 1 << bits, size=(T, 16))
        p = asym_pack(bits, codes, sb, zp)
        exact = ((codes.reshape(T, 16, AGROUP) - zp[:, :, None]) * f16_value(sb)[:, :, None]).ravel()
        assert np.array_equal(o.decode_f32(fid, p, T * 2048).astype(np.float64), exact), bits
        for dtype in DTYPES:
            want = f16_bits(exact) if dtype == "fp16" else bf16_bits(exact)
            assert np.array_equal(o.decode(fid, dtype, p, T * 2048), want), (bits, dtype)


def pin_asym_reduce_exact(o, seed=23):
    """Two ranks on the same group grid (scale s, zero point z) whose sums stay
    on it and reach both ends: the re-encoded sum has scale s and zero point z
    and decodes to the exact sum; also the 4-bit -> 8-bit mixed case."""
    rng = np.random.default_rng(seed)
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        z = (qmax + 1) // 2
        for dtype in DTYPES:
            ng = 32
            a = rng.integers(-z, qmax - z + 1, size=(ng, AGROUP))
            b = np.clip(rng.integers(-3, 4, size=(ng, AGROUP)), -z - a, qmax - z - a)
            a[:, :4] = [-z, qmax - z, 0, 0]
            b[:, :4] = [0, 0, -z, qmax - z]
            tot = a + b
            assert np.all((tot >= -z) & (tot <= qmax - z))
            s = 2.0 ** rng.integers(-6, 2, size=ng)
            ra = o.encode(fid, dtype, dtype_bits(dtype, (a * s[:, None]).ravel()))
            rb = o.encode(fid, dtype, dtype_bits(dtype, (b * s[:, None]).ravel()))
            out, y = o.reduce(fid, dtype, [ra, rb], ng * AGROUP)
            codes, sb, zp = asym_unpack(bits, out)
            assert np.array_equal(sb.ravel(), f16_bits(s)) and np.all(zp == z), (bits, dtype)
            assert np.array_equal(codes.reshape(ng, AGROUP), tot + z), (bits, dtype)
            assert np.array_equal(y, dtype_bits(dtype, (tot * s[:, None]).ravel())), (bits, dtype)
            if bits == 4:   # same inputs re-encoded with 8-bit codes: scale s*15/255, exact when representable
                out8, y8 = o.reduce_mixed(fid, ASYM[8], dtype, [ra, rb], ng * AGROUP)
                c8, s8, z8 = asym_unpack(8, out8)
                d8 = f16_value(f16_bits(s * 15 / 255))
                assert np.array_equal(s8.ravel(), f16_bits(s * 15 / 255)), dtype
                assert np.all(np.abs(dtype_value(dtype, y8) - (tot * s[:, None]).ravel())
                              <= np.repeat(d8, AGROUP) * 0.51 + np.abs((tot * s[:, None]).ravel()) * 2.0 ** -7)


def pin_asym_overflow_sum(o):
    """fp16 sums beyond the largest finite value round to +-inf (IEEE
    overflow).  In a group with +inf, hi = inf, so the scale saturates at 65504
    (0x7BFF); lo = 0 gives z = 0, and the code of +inf is rint(inf) + 0
    clamped to qmax; decode gives qmax * 65504, which is inf again in fp16.
    With -inf as well, -lo * e = inf clamps z to qmax and -inf codes to 0
    (decoding to -qmax * 65504 = -inf), while +inf codes to qmax = z and so
    decodes to 0."""
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        a = np.zeros(TILE)
        a[:AGROUP] = 1.0
        a[0:3] = 60000.0                              # + 60000 below -> 120000 -> +inf
        a[AGROUP:AGROUP + 2] = [60000.0, -60000.0]    # group 1: +inf and -inf
        b = np.zeros(TILE)
        b[0:3] = 60000.0
        b[AGROUP:AGROUP + 2] = [60000.0, -60000.0]
        ra = o.encode(fid, "fp16", f16_bits(a))
        rb = o.encode(fid, "fp16", f16_bits(b))
        out, y = o.reduce(fid, "fp16", [ra, rb], TILE)
        codes, sb, zp = asym_unpack(bits, out)
        assert sb[0, 0] == 0x7BFF and zp[0, 0] == 0, (bits, hex(sb[0, 0]), zp[0, 0])
        assert np.all(codes[0, 0:3] == qmax), (bits, codes[0, :3])
        assert sb[0, 1] == 0x7BFF and zp[0, 1] == qmax, (bits, zp[0, 1])
        assert codes[0, AGROUP] == qmax and codes[0, AGROUP + 1] == 0, (bits, codes[0, AGROUP:AGROUP + 2])
        assert np.all(y[0:3] == 0x7C00) and y[AGROUP] == 0 and y[AGROUP + 1] == 0xFC00, bits


def pin_asym_error_bound(o, seed=24):
    """|decode(encode(x)) - x| <= (0.5 + qmax * 2^-11) * s for every value: inside
    the grid the error is half a step; the fp16 rounding of the scale can leave
    the grid's top end short of the group maximum by up to qmax * 2^-11 steps,
    where the value clamps.  And the bound is not vacuous."""
    rng = np.random.default_rng(seed)
    for bits, fid in ASYM.items():
        for dtype in DTYPES:
            ng = 16 * 8
            x = rng.standard_normal((ng, AGROUP)) * np.exp(rng.uniform(-4, 4, (ng, 1))) + \
                rng.uniform(-2, 2, (ng, 1))
            xb = dtype_bits(dtype, x.astype(np.float32).astype(np.float64).ravel()) if dtype == "bf16" \
                else f16_bits(x.ravel())
            xv = dtype_value(dtype, xb)
            p = o.encode(fid, dtype, xb)
            y = o.decode_f32(fid, p, xv.size).astype(np.float64)
            _, sb, _ = asym_unpack(bits, p)
            s = np.repeat(f16_value(sb.ravel()), AGROUP)
            err = np.abs(y - xv)
            qmax = (1 << bits) - 1
            assert np.all(err <= (0.5 + qmax * 2.0 ** -11 + 1e-3) * s + 1e-30), (bits, dtype, (err / s).max())
            assert np.median(err / s) < 0.35


# ---------------------------------------------------------------------------
# P8: error bound of encode -> reduce -> decode against the exact sum
# ---------------------------------------------------------------------------

def _ulp(dtype, v):
    """Spacing of the dtype's values at |v| (normal and subnormal range)."""
    sig, emin = (11, -14) if dtype == "fp16" else (8, -126)
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** emin)))
    return 2.0 ** (e - (sig - 1))


def pin_error_bound(o, seed=8):
    rng = np.random.default_rng(seed)
    for bits in BITS:
        Q = qmax(bits)
        c = 1 + Q / 2048 + 1e-6        # worst case per value, in units of the block scale
        for dtype in DTYPES:
            for R in (1, 2, 4, 8):
                n = 2 * TILE
                xs = [_rng_blocks(rng, dtype, n // BLOCK, -3, 3) for _ in range(R)]
                xv = [dtype_value(dtype, xb) for xb in xs]
                ranks = [o.encode(bits, dtype, xb) for xb in xs]
                out, y = o.reduce(bits, dtype, ranks, n)
                exact = np.sum(xv, axis=0)
                d_in = [f16_value(unpack(bits, p)[1]).repeat(BLOCK, axis=1).ravel() for p in ranks]
                d_out = f16_value(unpack(bits, out)[1]).repeat(BLOCK, axis=1).ravel()
                absy = np.sum([np.abs(v) for v in xv], axis=0) + np.sum(d_in, axis=0) * Q
                e1 = c * np.sum(d_in, axis=0) + R * Q * 2.0 ** -24   # input quantization
                e2 = R * 2.0 ** -24 * absy                           # fp32 rank-order sum
                big = np.abs(exact) + e1 + e2
                e3 = _ulp(dtype, big)                                # sum rounded to dtype
                e4 = c * d_out + Q * 2.0 ** -24                      # re-quantization
                e5 = _ulp(dtype, big + e3 + e4)                      # output rounded to dtype
                bound = e1 + e2 + e3 + e4 + e5
                yv = dtype_value(dtype, y)
                err = np.abs(yv - exact)
                bad = err > bound
                assert not bad.any(), (bits, dtype, R, err[bad][:4], bound[bad][:4])
                # and the bound is not vacuous: the error is typically far below it
                assert np.median(err / bound) < 0.6



def pin_asym_zero_point_clamp(o):
    """The zero point is clamped to [0, 2^b - 1] where rounding of the scale
    pushes -lo / s past the top code.  Hand-derived cases:
      * fp16, range [-k * 2^-24, 0] with k = 22 (4-bit) or 357 (8-bit):
        t = k / qmax * 2^-24 rounds to the smallest subnormal 2^-24 (ratio 1.47,
        1.40 < 1.5), so -lo / s = k > qmax and z = qmax; the minimum then
        clamps to code 0 and zeros encode as z.
      * bf16, range [-2^30, 0]: t = 2^30 / qmax > 65504 saturates the scale
        at 65504 (0x7BFF), -lo / s = 2^30 / 65504 > 16000 and z = qmax."""
    for bits, fid in ASYM.items():
        qmax = (1 << bits) - 1
        k = 22 if bits == 4 else 357
        cases = [("fp16", -k * 2.0 ** -24, 0x0001), ("bf16", -2.0 ** 30, 0x7BFF)]
        for dtype, lo, want_sb in cases:
            x = np.zeros(TILE)
            x[0] = lo
            p = o.encode(fid, dtype, dtype_bits(dtype, x))
            codes, sb, zp = asym_unpack(bits, p)
            assert sb[0, 0] == want_sb and zp[0, 0] == qmax, (bits, dtype, sb[0, 0], zp[0, 0])
            assert codes[0, 0] == 0 and np.all(codes[0, 1:AGROUP] == qmax), (bits, dtype)
            y = dtype_value(dtype, o.decode(fid, dtype, p, TILE))
            assert np.all(y[1:] == 0), (bits, dtype)
            want = -qmax * float(f16_value(np.uint16(want_sb)))   # exact, then rounded to the dtype
            assert y[0] == dtype_value(dtype, dtype_bits(dtype, np.array([want])))[0], (bits, dtype)



# ---------------------------------------------------------------------------
# FP4 E2M1 block codec (format id 36, laid out like INT4)
# ---------------------------------------------------------------------------

FP4 = 36
FP4_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def fp4_nearest(v):
    """E2M1 code nearest to each float64 v by brute-force distance over the
    eight magnitudes, a tie going to the code with an even mantissa bit;
    magnitudes above 6 take 6; the sign bit is v's sign (-0 and negative
    values that round to zero give code 8)."""
    v = np.asarray(v, np.float64)
    a = np.minimum(np.abs(v), 6.0)
    dist = np.abs(a[:, None] - FP4_MAG[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(8)[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return pick + 8 * np.signbit(v)


def pin_fp4_value_table(o):
    """Decoding codes 0..15 with scale 1.0 gives the E2M1 values of the OCP MX
    specification (golden fp4_e2m1_values.txt); the code sits in the INT4
    nibble order and the scale in the INT4 scale slot."""
    rows = read_golden("fp4_e2m1_values.txt")
    want = {int(r[0]): float(r[4]) for r in rows}
    neg_zero = {int(r[0]) for r in rows if r[4] == "-0"}
    codes = np.tile(np.arange(16), 2048 // 16).reshape(1, 2048)
    sb = np.full((1, 64), 0x3C00, np.uint16)
    y = o.decode_f32(FP4, pack(4, codes, sb), 2048)
    for i in range(32):
        c = int(codes[0, i])
        assert y[i] == want[c], (c, y[i], want[c])
        assert np.signbit(y[i]) == (c in neg_zero or want[c] < 0), c
    assert o.packed_bytes(FP4, 2048) == 1152


def _fp4_blocks(anchor, xs):
    """Blocks [anchor, x, 0, ...] as fp16 bits, padded to whole tiles."""
    nb = xs.size
    blocks = np.zeros((nb, BLOCK), np.uint16)
    blocks[:, 0] = f16_bits(anchor)
    blocks[:, 1] = f16_bits(xs)
    return pad_tiles(blocks), nb


def pin_fp4_bruteforce_pow2(o):
    """Blocks [6 * 2^k, x, 0...]: the scale is 2^k exactly (6 * 2^k / 6) and
    the code of every finite fp16 x with |x| <= 6 * 2^k is the E2M1 value
    nearest to x / 2^k (brute-force distance, ties to an even mantissa,
    sign kept), for exponents k covering normal and subnormal fp16 scales;
    decode gives that value times 2^k."""
    allb, allv = all_finite("fp16")
    for k in (-24, -20, -14, -6, -1, 0, 3, 12):
        a = 6.0 * 2.0 ** k
        if f16_value(f16_bits(a)) != a:
            continue
        sel = np.abs(allv) <= a
        xv = allv[sel]
        p, nb = _fp4_blocks(a, xv)
        codes, sb = unpack(4, o.encode(FP4, "fp16", p))
        codes = codes.reshape(-1, BLOCK)[:nb]
        assert np.all(sb.ravel()[:nb] == pow2_f16_bits(k)), k
        want = fp4_nearest(xv / 2.0 ** k)
        bad = codes[:, 1] != want
        assert not bad.any(), (k, xv[bad][:4], codes[bad, 1][:4], want[bad][:4])
        assert np.all(codes[:, 0] == 7), k
        y = o.decode_f32(FP4, o.encode(FP4, "fp16", p), p.size).reshape(-1, BLOCK)[:nb, 1]
        vals = np.where(want >= 8, -FP4_MAG[want % 8], FP4_MAG[want % 8]) * 2.0 ** k
        assert np.array_equal(y.astype(np.float64), vals), k


def pin_fp4_general_scale(o):
    """Non-power-of-two scales d with 6 * d exact in fp16: the scale is d and
    the code of every fp16 x in range is the nearest E2M1 value to
    RN32(x * RN32(1/d)) (products in float64, rounded once).  Some x round
    differently under x / d, so the pin separates multiplying by the fp32
    reciprocal from dividing by the scale."""
    allb, allv = all_finite("fp16")
    diff_seen = 0
    for d_bits in (0x3555, 0x2E66, 0x3A00, 0x0F90, 0x3300, 0x3368, 0x17A8, 0x3480):
        d = float(f16_value(np.uint16(d_bits)))
        a = 6.0 * d
        if f16_value(f16_bits(a)) != a:
            continue
        xv = allv[np.abs(allv) <= a]
        p, nb = _fp4_blocks(a, xv)
        codes, sb = unpack(4, o.encode(FP4, "fp16", p))
        codes = codes.reshape(-1, BLOCK)[:nb]
        assert np.all(sb.ravel()[:nb] == d_bits), hex(d_bits)
        e = np.float64(np.float32(1.0 / d))
        v = (xv * e).astype(np.float32).astype(np.float64)
        want = fp4_nearest(v)
        bad = codes[:, 1] != want
        assert not bad.any(), (hex(d_bits), xv[bad][:4], codes[bad, 1][:4], want[bad][:4])
        diff_seen += int((fp4_nearest((xv / d).astype(np.float32).astype(np.float64)) != want).sum())
    assert diff_seen > 0


def pin_fp4_scale_every_max(o):
    """For every positive finite fp16 block maximum m (block [m, 0, ...]): the
    scale is fp16(RN32(m / 6)), the quotient taken in float64 and rounded once
    to float32 (harmless double rounding: 53 >= 2 * 24 + 2) and then to fp16;
    the maximum itself codes as 6 (or saturates).  (m * RN32(1/6) differs from
    RN32(m / 6) for about a third of the m, by one fp32 ulp, but never after
    the rounding to fp16, for any fp16 or bf16 m: the two readings give the
    same scale, so no planted mistake can separate them.)"""
    m_bits = np.arange(1, 0x7C00, dtype=np.uint16)
    m = f16_value(m_bits).astype(np.float64)
    p, nb = _fp4_blocks(0.0, np.zeros(0))
    blocks = np.zeros((m.size, BLOCK), np.uint16)
    blocks[:, 0] = m_bits
    codes, sb = unpack(4, o.encode(FP4, "fp16", pad_tiles(blocks)))
    t = (m / 6.0).astype(np.float32)
    want = f16_bits(np.minimum(t.astype(np.float64), 65504.0))
    got = sb.ravel()[:m.size]
    assert np.array_equal(got, want), np.argwhere(got != want)[:4].ravel().tolist()
    d = f16_value(got).astype(np.float64)
    ok = d > 0
    e = (1.0 / d[ok]).astype(np.float32).astype(np.float64)
    v = (m[ok] * e).astype(np.float32).astype(np.float64)
    assert np.array_equal(codes.reshape(-1, BLOCK)[:m.size, 0][ok], fp4_nearest(v))


def pin_fp4_zero_and_saturation(o):
    """Zero and -0 blocks: scale 0, codes 0 and 8 (sign kept), decode +-0.
    A bf16 block whose maximum exceeds 6 * 65504: the scale saturates at
    65504 (0x7BFF) and values beyond 6 * 65504 code as +-6 (7 / 15)."""
    for dtype in DTYPES:
        x = np.zeros(2048)
        x[32:64:2] = -0.0
        x[64:96] = 0.0
        x[64] = -2.0 ** -100 if dtype == "bf16" else 0.0   # scale rounds to 0: x * 0 = -0
        codes, sb = unpack(4, o.encode(FP4, dtype, dtype_bits(dtype, x)))
        assert sb[0, 0] == 0 and sb[0, 1] == 0 and np.all(codes[0, :32] == 0)
        assert np.all(codes[0, 32:64:2] == 8) and np.all(codes[0, 33:64:2] == 0)
        if dtype == "bf16":
            assert codes[0, 64] == 8
    xb = np.zeros(2048)
    xb[:4] = [2.0 ** 30, -2.0 ** 30, 3.0 * 65504, -1.0]
    codes, sb = unpack(4, o.encode(FP4, "bf16", bf16_bits(xb)))
    assert sb[0, 0] == 0x7BFF
    assert codes[0, 0] == 7 and codes[0, 1] == 15
    assert codes[0, 2] == fp4_nearest([float(np.float32(np.float32(bf16_value(bf16_bits(3.0 * 65504))) * np.float32(1 / 65504.0)))])[0]


def pin_fp4_reduce_exact(o, seed=31):
    """Two ranks whose blocks share the scale s (a 6 * s anchor in each, at
    positions where the other rank is 0) and whose element pairs sum to E2M1
    values: the re-encoded sum has scale s, the exact codes, and decodes to
    the exact sum."""
    rng = np.random.default_rng(seed)
    pairs = [(0.5, 0.5, 1.0), (1, 1, 2), (1.5, 1.5, 3), (2, 2, 4), (3, 3, 6), (0.5, 1, 1.5),
             (-1, 3, 2), (4, -1, 3), (-2, -1, -3), (-0.5, -1, -1.5), (2, -6, -4), (0, 0, 0), (6, -6, 0)]
    for dtype in DTYPES:
        nb = 64
        a = np.zeros((nb, BLOCK)); b = np.zeros((nb, BLOCK)); tot = np.zeros((nb, BLOCK))
        idx = rng.integers(0, len(pairs), size=(nb, BLOCK))
        for j, (pa, pb, pt) in enumerate(pairs):
            a[idx == j], b[idx == j], tot[idx == j] = pa, pb, pt
        a[:, 0], b[:, 0], tot[:, 0] = 6, 0, 6
        a[:, 1], b[:, 1], tot[:, 1] = 0, 6, 6
        s = 2.0 ** rng.integers(-8, 3, size=nb)
        ra = o.encode(FP4, dtype, dtype_bits(dtype, (a * s[:, None]).ravel()))
        rb = o.encode(FP4, dtype, dtype_bits(dtype, (b * s[:, None]).ravel()))
        out, y = o.reduce(FP4, dtype, [ra, rb], nb * BLOCK)
        codes, sb = unpack(4, out)
        assert np.array_equal(sb.ravel(), f16_bits(s)), dtype
        assert np.array_equal(codes.reshape(nb, BLOCK), fp4_nearest(tot.ravel()).reshape(nb, BLOCK)), dtype
        assert np.array_equal(y, dtype_bits(dtype, (tot * s[:, None]).ravel())), dtype


def _fp4_exact(codes, sb):
    """Exact decode in float64 from the E2M1 magnitudes and the block scales."""
    c = np.asarray(codes).reshape(-1, 64, BLOCK)
    mag = FP4_MAG[c % 8] * f16_value(sb)[:, :, None]
    return np.where(c >= 8, -mag, mag).ravel()


def pin_fp4_reduce_r1_composition(o, seed=32):
    """R = 1: the reduce re-encodes dtype_RNE(exact decode) and decodes it; the
    exact decode and the dtype rounding are computed here in numpy / torch
    from the codes and scales."""
    rng = np.random.default_rng(seed)
    for dtype in DTYPES:
        n = 2 * TILE
        xb = _rng_blocks(rng, dtype, n // BLOCK)
        p = o.encode(FP4, dtype, xb)
        codes, sb = unpack(4, p)
        zb = dtype_bits(dtype, _fp4_exact(codes, sb))
        out, y = o.reduce(FP4, dtype, [p], n)
        assert np.array_equal(out, o.encode(FP4, dtype, zb)), dtype
        c2, s2 = unpack(4, out)
        assert np.array_equal(y, dtype_bits(dtype, _fp4_exact(c2, s2))), dtype


def pin_fp4_error_bound(o, seed=33):
    """|decode(encode(x)) - x| is at most half the E2M1 spacing at x / d (0.25,
    0.5 or 1 times d) plus the effect of the rounded scale, per value; the
    bound is reached to within 10% on random data (not vacuous)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(64 * 2048)
    xb = f16_bits(x)
    xv = f16_value(xb).astype(np.float64)
    p = o.encode(FP4, "fp16", xb)
    codes, sb = unpack(4, p)
    d = np.repeat(f16_value(sb.ravel()).astype(np.float64), 32)
    y = o.decode_f32(FP4, p, x.size).astype(np.float64)
    a = np.abs(xv) / d
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0))
    bound = half * d + np.abs(xv) * 2.0 ** -10 + 1e-30
    err = np.abs(y - xv)
    assert np.all(err <= bound), float((err / bound).max())
    assert (err / bound).max() > 0.9

ALL_PINS = [
    pin_tile_bytes,
    pin_unit_bit_order,
    pin_scale_placement,
    pin_exact_roundtrip,
    pin_extremes_and_grid,
    pin_zero_tiny_huge,
    pin_bruteforce_pow2,
    pin_bruteforce_general_scale,
    pin_scale_reciprocal_exhaustive,
    pin_f16_conversions,
    pin_bf16_conversions,
    pin_decode_rounding,
    pin_reduce_r1_composition,
    pin_reduce_exact_common_scale,
    pin_reduce_rank_order,
    pin_reduce_exact_terms,
    pin_reduce_mixed_r1_composition,
    pin_reduce_mixed_exact,
    pin_asym_tile_layout,
    pin_asym_exact_roundtrip,
    pin_asym_bruteforce_pow2,
    pin_asym_bruteforce_general_scale,
    pin_asym_group_params,
    pin_asym_special_groups,
    pin_asym_decode_algorithm1,
    pin_asym_reduce_exact,
    pin_asym_zero_point_clamp,
    pin_asym_overflow_sum,
    pin_asym_error_bound,
    pin_error_bound,
    pin_fp4_value_table,
    pin_fp4_bruteforce_pow2,
    pin_fp4_general_scale,
    pin_fp4_scale_every_max,
    pin_fp4_zero_and_saturation,
    pin_fp4_reduce_exact,
    pin_fp4_reduce_r1_composition,
    pin_fp4_error_bound,
]

