"""The CPU oracle against its pins (page values, closed forms, invariants)."""
import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=[p.__name__ for p in P.ALL_PINS])
def test_pin(oracle, pin):
    pin(oracle)


def test_float64_formulation(oracle):
    """Cross-check (not a pin): random blocks against a float64 formulation of the
    same steps, each binary32 rounding done by numpy.  A product of two float32
    values is exact in float64, so rounding it once to float32 is RN32."""
    rng = np.random.default_rng(11)
    for bits in P.BITS:
        Q = P.qmax(bits)
        for dtype in P.DTYPES:
            nb = 64 * 8
            xb = P._rng_blocks(rng, dtype, nb, -8, 8)
            xv = P.dtype_value(dtype, xb).reshape(nb, P.BLOCK)
            m = np.abs(xv).max(axis=1)
            t = np.minimum(m / Q, 65504.0)
            d = P.f16_value(P.f16_bits(t))
            e = np.where(d == 0, 0.0, (1.0 / np.where(d == 0, 1.0, d)).astype(np.float32).astype(np.float64))
            v = (xv * e[:, None]).astype(np.float32).astype(np.float64)
            k = np.rint(np.clip(v, -Q, Q - 1))
            p = oracle.encode(bits, dtype, xb)
            codes, sb = P.unpack(bits, p)
            assert np.array_equal(codes.reshape(nb, P.BLOCK), k + Q), (bits, dtype)
            assert np.array_equal(sb.ravel(), P.f16_bits(d)), (bits, dtype)
