"""The C oracle against an independent numpy model of the same rules.

A cross-check, not a pin (the pins are in ``oracle_pins.py``): both sides
restate the codec, so agreement rules out slips in either one but not a
reading that both share.  Every entry point is compared byte for byte on
inputs built to reach every branch: ordinary and heavy-tailed activations,
blocks spread over the whole exponent range of the I/O dtype, exact ties of
the rounding, zero, single-value and saturating blocks, and sums that
overflow binary16.
"""
import numpy as np
import pytest

import model_f64 as M
import oracle_pins as P

FORMATS = (3, 4, 8, 20, 24, 36)
MIXED = ((4, 8), (8, 4), (3, 8), (8, 3), (3, 4), (20, 24), (24, 20))
TILES = 6


def _finite_bits(dtype, x):
    """dtype bits of float64 values, clipped first to a finite range of the dtype."""
    top = 65504.0 if dtype == "fp16" else 3.0e38
    with np.errstate(over="ignore"):
        x = np.clip(np.asarray(x, np.float64), -top, top).astype(np.float32).astype(np.float64)
    return P.dtype_bits(dtype, x)


FP4_MIDPOINTS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _ties(rng, n):
    """Groups of 128 values that put x * e exactly halfway between two codes.
    Each group takes one of six shapes, for one of the formats: symmetric
    blocks whose maximum is Q * 2^k (scale 2^k) holding (j + 1/2) * 2^k;
    FP4 blocks with maximum 6 * 2^k holding midpoints of E2M1 values times
    2^k; asymmetric groups spanning [-z0 * 2^k, (2^b - 1 - z0) * 2^k] (scale
    2^k, zero point z0) holding (j + 1/2) * 2^k."""
    x = np.zeros((n // 128, 128))
    for g in range(n // 128):
        shape = rng.integers(6)
        if shape < 3:
            Q = (4, 8, 128)[shape]
            for blk in range(4):
                k = float(rng.integers(-10, 4))
                v = (rng.integers(-Q, Q, 32) + 0.5) * 2.0 ** k
                v[rng.integers(32)] = rng.choice([-1.0, 1.0]) * Q * 2.0 ** k
                x[g, 32 * blk:32 * blk + 32] = v
        elif shape == 3:
            for blk in range(4):
                k = float(rng.integers(-10, 10))
                v = rng.choice([-1.0, 1.0], 32) * rng.choice(FP4_MIDPOINTS, 32) * 2.0 ** k
                v[rng.integers(32)] = 6 * 2.0 ** k
                x[g, 32 * blk:32 * blk + 32] = v
        else:
            qm = 15 if shape == 4 else 255
            k = float(rng.integers(-10, 4))
            z0 = int(rng.integers(1, qm))
            v = (rng.integers(-z0, qm - z0, 128) + 0.5) * 2.0 ** k
            i, j = rng.choice(128, 2, replace=False)
            v[i], v[j] = -z0 * 2.0 ** k, (qm - z0) * 2.0 ** k
            x[g] = v
    return x


def family(name, dtype, rng, tiles=TILES):
    """uint16 bit patterns (tiles * 2048 values) of one input family."""
    n = tiles * 2048
    lo_exp, hi_exp = (-24, 15) if dtype == "fp16" else (-133, 127)
    if name == "normal_outliers":
        x = rng.standard_normal(n)
        x[rng.random(n) < 1e-3] *= 50
    elif name == "exponent_sweep":
        # every 32-value block has its own scale 2^k over the dtype's whole range
        k = rng.integers(lo_exp, hi_exp, size=n // 32)
        x = rng.standard_normal((n // 32, 32)) * np.exp2(k.astype(np.float64))[:, None]
    elif name == "ties":
        x = _ties(rng, n)
    elif name == "sparse_special":
        x = np.zeros((n // 32, 32))
        kinds = rng.integers(0, 5, size=n // 32)
        for b, kind in enumerate(kinds):
            if kind == 1:        # one nonzero value
                x[b, rng.integers(32)] = rng.standard_normal()
            elif kind == 2:      # the largest finite values of the dtype
                x[b] = rng.choice([-1.0, 1.0], 32) * (65504.0 if dtype == "fp16" else 3.0e38)
            elif kind == 3:      # smallest subnormals
                x[b] = rng.integers(-3, 4, 32) * np.exp2(lo_exp)
            elif kind == 4:      # all negative, so the maximum comes from the minimum
                x[b] = -np.abs(rng.standard_normal(32))
    else:
        raise ValueError(name)
    return _finite_bits(dtype, x.ravel())


FAMILIES = ("normal_outliers", "exponent_sweep", "ties", "sparse_special")


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_encode_decode_match_model(oracle, fmt, dtype):
    rng = np.random.default_rng(100 + fmt)
    for name in FAMILIES:
        xb = family(name, dtype, rng)
        p = oracle.encode(fmt, dtype, xb)
        assert np.array_equal(p, M.encode(fmt, dtype, xb)), (fmt, dtype, name, "encode")
        n = xb.size
        yf = oracle.decode_f32(fmt, p, n).astype(np.float64)
        ym = M.decode_f32(fmt, p, n)
        assert np.array_equal(yf, ym) and np.array_equal(np.signbit(yf), np.signbit(ym)), \
            (fmt, dtype, name, "decode_f32")
        assert np.array_equal(oracle.decode(fmt, dtype, p, n), M.decode(fmt, dtype, p, n)), \
            (fmt, dtype, name, "decode")


@pytest.mark.parametrize("dtype", P.DTYPES)
@pytest.mark.parametrize("fmt", FORMATS)
def test_reduce_matches_model(oracle, fmt, dtype):
    rng = np.random.default_rng(200 + fmt)
    for R in (1, 2, 3, 8, 16):
        for name in FAMILIES:
            ranks = [oracle.encode(fmt, dtype, family(name, dtype, rng, tiles=2)) for _ in range(R)]
            n = 2 * 2048
            po, yo = oracle.reduce(fmt, dtype, ranks, n)
            pm, ym = M.reduce_mixed(fmt, fmt, dtype, ranks, n)
            assert np.array_equal(po, pm), (fmt, dtype, R, name, "packed_out")
            assert np.array_equal(yo, ym), (fmt, dtype, R, name, "y_out")


@pytest.mark.parametrize("fmt_in,fmt_out", MIXED)
def test_mixed_reduce_matches_model(oracle, fmt_in, fmt_out):
    rng = np.random.default_rng(300 + 10 * fmt_in + fmt_out)
    for dtype in P.DTYPES:
        for name in FAMILIES:
            ranks = [oracle.encode(fmt_in, dtype, family(name, dtype, rng, tiles=2)) for _ in range(4)]
            po, yo = oracle.reduce_mixed(fmt_in, fmt_out, dtype, ranks, 4096)
            pm, ym = M.reduce_mixed(fmt_in, fmt_out, dtype, ranks, 4096)
            assert np.array_equal(po, pm), (fmt_in, fmt_out, dtype, name)
            assert np.array_equal(yo, ym), (fmt_in, fmt_out, dtype, name)


def test_fp16_sum_overflow_matches_model(oracle):
    """Eight ranks of values near the binary16 maximum: the binary32 sum
    rounds to +-inf in binary16, and the re-encode of that block saturates."""
    rng = np.random.default_rng(7)
    for fmt in FORMATS:
        ranks = []
        for _ in range(8):
            x = rng.choice([-1.0, 1.0], 2048) * rng.uniform(30000, 65504, 2048)
            x[:1024] = np.abs(x[:1024])
            ranks.append(oracle.encode(fmt, "fp16", _finite_bits("fp16", x)))
        po, yo = oracle.reduce(fmt, "fp16", ranks, 2048)
        pm, ym = M.reduce_mixed(fmt, fmt, "fp16", ranks, 2048)
        assert np.array_equal(po, pm), fmt
        assert np.array_equal(yo, ym), fmt
