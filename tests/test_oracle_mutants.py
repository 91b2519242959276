"""Planted mistakes in the oracle must fail at least one pin.

Each mutant copies ``oracle/qr_oracle.c`` into a temporary directory, applies one
plausible mistake (a dropped term, a wrong sign, index, bound, rounding or
order), builds it with the same flags and runs the pins of ``oracle_pins``
against it.  The real oracle passes every pin (``test_oracle_pins.py``); a
mutant that passes them all means the pins have a blind spot.  Everything here
runs on the CPU.
"""

import pytest

import oracle
import oracle.build as obuild
import oracle_pins as P

SRC = obuild.SRC

# (name, [(old, new), ...]) -- every `old` must occur exactly once in the source.
MUTANTS = [
    ("bias dropped", [("codes[i] = (unsigned)(k + Q);", "codes[i] = (unsigned)(k + Q - 1);")]),
    ("scale divides by Q-1", [("float t = m / (float)Q; ", "float t = m / (float)(Q - 1); ")]),
    ("round half away from zero", [("long k = lrintf(c);", "long k = lroundf(c);")]),
    ("truncate instead of round", [("long k = lrintf(c);", "long k = (long)c;")]),
    ("clip top at Q", [("float c = fminf(fmaxf(v, -(float)Q), (float)(Q - 1));",
                        "float c = fminf(fmaxf(v, -(float)Q), (float)Q);")]),
    ("clip bottom at -(Q-1)", [("float c = fminf(fmaxf(v, -(float)Q), (float)(Q - 1));",
                                "float c = fminf(fmaxf(v, -(float)(Q - 1)), (float)(Q - 1));")]),
    ("no clip", [("float c = fminf(fmaxf(v, -(float)Q), (float)(Q - 1));", "float c = v;")]),
    ("INT4 nibble order reversed", [
        ("w |= (uint32_t)code << (4 * j);", "w |= (uint32_t)code << (4 * (7 - j));"),
        ("return (w >> (4 * j)) & 15u;", "return (w >> (4 * (7 - j))) & 15u;")]),
    ("INT3 1-bit plane order reversed", [
        ("(uint8_t)(((code >> 2) & 1u) << j);", "(uint8_t)(((code >> 2) & 1u) << (7 - j));"),
        ("unsigned high = (tile[INT3_Q1_OFFSET + u] >> j) & 1u;",
         "unsigned high = (tile[INT3_Q1_OFFSET + u] >> (7 - j)) & 1u;")]),
    ("INT3 split high-two / low-one", [
        ("w |= (code & 3u) << (2 * j);", "w |= (code >> 1) << (2 * j);"),
        ("(uint8_t)(((code >> 2) & 1u) << j);", "(uint8_t)((code & 1u) << j);"),
        ("return low | (high << 2);", "return (low << 1) | high;")]),
    ("INT3 planes swapped", [
        ("#define INT3_Q1_OFFSET 512", "#define INT3_Q1_OFFSET 0"),
        ("unsigned w = tile[2 * u] | (tile[2 * u + 1] << 8);\n    w |= (code & 3u) << (2 * j);\n"
         "    tile[2 * u] = (uint8_t)(w & 0xff);\n    tile[2 * u + 1] = (uint8_t)(w >> 8);",
         "unsigned w = tile[256 + 2 * u] | (tile[256 + 2 * u + 1] << 8);\n    w |= (code & 3u) << (2 * j);\n"
         "    tile[256 + 2 * u] = (uint8_t)(w & 0xff);\n    tile[256 + 2 * u + 1] = (uint8_t)(w >> 8);"),
        ("unsigned w = tile[2 * u] | (tile[2 * u + 1] << 8);\n    unsigned low",
         "unsigned w = tile[256 + 2 * u] | (tile[256 + 2 * u + 1] << 8);\n    unsigned low")]),
    ("scale stored big-endian", [
        ("p[0] = (uint8_t)(d & 0xff);\n  p[1] = (uint8_t)(d >> 8);",
         "p[1] = (uint8_t)(d & 0xff);\n  p[0] = (uint8_t)(d >> 8);"),
        ("return (uint16_t)(p[0] | (p[1] << 8));", "return (uint16_t)(p[1] | (p[0] << 8));")]),
    ("scale not saturated at 65504", [("if (t > 65504.0f) t = 65504.0f; /* largest finite binary16 */", "")]),
    ("multiplier rounded to fp16", [("*e = (d == 0.0f) ? 0.0f : 1.0f / d;\n}",
                                     "*e = (d == 0.0f) ? 0.0f : qro_f16_to_f32(qro_f32_to_f16(1.0f / d));\n}")]),
    ("multiplier from the block maximum", [("*e = (d == 0.0f) ? 0.0f : 1.0f / d;\n}",
                                            "*e = (d == 0.0f) ? 0.0f : (float)Q / m;\n}")]),
    ("divide by the scale", [("float v = x[i] * e;",
                              "float v = (e == 0.0f) ? 0.0f : x[i] / qro_f16_to_f32(*d_bits);")]),
    ("signed maximum", [("float a = fabsf(x[i]);", "float a = x[i];")]),
    ("decode bias dropped", [("return (float)((int)code - Q) * d;", "return (float)((int)code - Q + 1) * d;")]),
    ("decode sign flipped", [("return (float)((int)code - Q) * d;", "return (float)(Q - (int)code) * d;")]),
    ("rank order reversed", [
        ("float s = decode_value_fmt(fmt_in, ranks[0] + t * tb, i);\n"
         "      for (int r = 1; r < R; ++r) s = s + decode_value_fmt(fmt_in, ranks[r] + t * tb, i);",
         "float s = decode_value_fmt(fmt_in, ranks[R - 1] + t * tb, i);\n"
         "      for (int r = R - 2; r >= 0; --r) s = s + decode_value_fmt(fmt_in, ranks[r] + t * tb, i);")]),
    ("rank 0 dropped", [("float s = decode_value_fmt(fmt_in, ranks[0] + t * tb, i);", "float s = 0.0f;")]),
    ("last rank dropped", [("for (int r = 1; r < R; ++r) s = s +", "for (int r = 1; r < R - 1; ++r) s = s +")]),
    ("sum in double", [
        ("float s = decode_value_fmt(fmt_in, ranks[0] + t * tb, i);",
         "double s = decode_value_fmt(fmt_in, ranks[0] + t * tb, i);"),
        ("z[i] = dtype_to_f32(dtype, f32_to_dtype(dtype, s));",
         "z[i] = dtype_to_f32(dtype, f32_to_dtype(dtype, (float)s));")]),
    ("sum not rounded to dtype", [("z[i] = dtype_to_f32(dtype, f32_to_dtype(dtype, s));", "z[i] = s;")]),
    ("terms rounded to dtype", [("s = s + decode_value_fmt(fmt_in, ranks[r] + t * tb, i);",
                                 "s = s + dtype_to_f32(dtype, f32_to_dtype(dtype, decode_value_fmt(fmt_in, ranks[r] + t * tb, i)));")]),
    ("fp16 ties away from zero", [("  float r = rintf(a / quantum) * quantum;\n  if (r < 0x1p-14f)",
                                   "  float r = roundf(a / quantum) * quantum;\n  if (r < 0x1p-14f)")]),
    ("bf16 truncation", [("float r = rintf(a / quantum) * quantum; /* exact scaling, ties to even */",
                          "float r = floorf(a / quantum) * quantum;")]),
    ("fp16 overflow at 65504", [("if (a >= 65520.0f)", "if (a > 65504.0f)")]),
    ("fp16 subnormal decode scale", [("mag = ldexpf((float)frac, -24);", "mag = ldexpf((float)frac, -25);")]),
    ("block of 16 values", [("#define QRO_BLOCK 32 ", "#define QRO_BLOCK 16 ")]),
    ("output decoded before re-encode", [
        ("y_out[t * QRO_TILE + i] = f32_to_dtype(dtype, decode_value_fmt(fmt_out, out, i));",
         "y_out[t * QRO_TILE + i] = f32_to_dtype(dtype, z[i]);")]),
    ("mixed: re-encode in the input format", [("encode_tile_fmt(fmt_out, z, out);", "encode_tile_fmt(fmt_in, z, out);")]),
    ("mixed: final decode in the input format", [
        ("y_out[t * QRO_TILE + i] = f32_to_dtype(dtype, decode_value_fmt(fmt_out, out, i));",
         "y_out[t * QRO_TILE + i] = f32_to_dtype(dtype, decode_value_fmt(fmt_in, out, i));")]),
    ("asym: range excludes zero", [("float lo = 0.0f, hi = 0.0f; /* the range always includes 0 */",
                                    "float lo = x[0], hi = x[0];")]),
    ("asym: divides the range by 2^b", [("float t = (hi - lo) / (float)qmax;", "float t = (hi - lo) / (float)(qmax + 1);")]),
    ("asym: zero point not added", [("float k = rintf(u) + (float)*z;", "float k = rintf(u);")]),
    ("asym: decode ignores the zero point", [("return (float)((int)get_code(bits, tile, i) - z) * d;",
                                              "return (float)((int)get_code(bits, tile, i)) * d;")]),
    ("asym: zero point not clamped", [("zf = fminf(fmaxf(zf, 0.0f), (float)qmax);", "")]),
    ("asym: codes clamp at qmax - 1", [("k = fminf(fmaxf(k, 0.0f), (float)qmax);", "k = fminf(fmaxf(k, 0.0f), (float)(qmax - 1));")]),
    ("asym: zero points overlap the codes", [("asym_scale_offset(bits) + 2 * QRO_AGROUPS; }",
                                              "asym_scale_offset(bits) - QRO_AGROUPS; }")]),
    ("asym: group scale not saturated", [("if (t > 65504.0f) t = 65504.0f; /* saturate the group scale */", "")]),
    ("asym: multiplier rounded to fp16", [("*e = (d == 0.0f) ? 0.0f : 1.0f / d; /* group multiplier */",
                                           "*e = (d == 0.0f) ? 0.0f : qro_f16_to_f32(qro_f32_to_f16(1.0f / d));")]),
    ("asym: divide by the scale", [("float u = x[i] * e;",
                                    "float u = (e == 0.0f) ? 0.0f : x[i] / qro_f16_to_f32(*d_bits);")]),
    ("asym: zero point truncated", [("float zf = rintf(-lo * *e);", "float zf = truncf(-lo * *e);")]),
    ("asym: no clamp at the top", [("k = fminf(fmaxf(k, 0.0f), (float)qmax);", "k = fmaxf(k, 0.0f);")]),
    ("asym: rounding after the zero point", [("float k = rintf(u) + (float)*z;", "float k = rintf(u + (float)*z);")]),
    ("fp4: ties away from zero", [("float r = rintf(a / step) * step; /* exact: the step is a power of two */",
                                  "float r = roundf(a / step) * step;")]),
    ("fp4: truncation", [("float r = rintf(a / step) * step; /* exact: the step is a power of two */",
                          "float r = floorf(a / step) * step;")]),
    ("fp4: saturation at 4", [("if (r > 6.0f) r = 6.0f;", "if (r > 4.0f) r = 4.0f;")]),
    ("fp4: maximum mapped to 4", [("float t = m / 6.0f; ", "float t = m / 4.0f; ")]),
    ("fp4: sign of zero dropped", [("return (signbit(v) ? 8u : 0u) | mc;", "return (v < 0.0f ? 8u : 0u) | mc;")]),
    ("fp4: exponent bias 2", [("ldexpf(1.0f + 0.5f * (float)m, ef - 1)", "ldexpf(1.0f + 0.5f * (float)m, ef - 2)")]),
    ("fp4: no subnormal", [("ef == 0 ? 0.5f * (float)m :", "ef == 0 ? 0.0f * (float)m :")]),
    ("fp4: uniform step 0.5", [("float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);", "float step = 0.5f;")]),
    ("fp4: divide by the scale", [("fp4_code(xb[i] * e)", "fp4_code(e == 0.0f ? 0.0f * xb[i] : xb[i] / qro_f16_to_f32(d_bits))")]),
    ("fp4: scale not saturated", [("if (t > 65504.0f) t = 65504.0f; /* saturate at the largest binary16 */", "")]),
    ("fp4: multiplier rounded to fp16", [("*e = (d == 0.0f) ? 0.0f : 1.0f / d; /* FP4 multiplier */",
                                          "*e = (d == 0.0f) ? 0.0f : qro_f16_to_f32(qro_f32_to_f16(1.0f / d));")]),
    ("fp4: decoded as INT4", [("if (fmt_fp4(fmt)) return decode_value_fp4(tile, i);", "")]),
    ("asym: groups of 64", [("#define QRO_AGROUP 128 ", "#define QRO_AGROUP 64 ")]),
]


# Pins that take a second or so on the real oracle run last against a mutant:
# the order changes only how soon a mutant is caught, not whether it is.
SLOW_PINS = {"pin_asym_bruteforce_general_scale", "pin_unit_bit_order", "pin_bruteforce_pow2",
             "pin_reduce_exact_common_scale", "pin_asym_bruteforce_pow2", "pin_bruteforce_general_scale",
             "pin_fp4_bruteforce_pow2", "pin_scale_reciprocal_exhaustive"}
PIN_ORDER = ([p for p in P.ALL_PINS if p.__name__ not in SLOW_PINS]
             + [p for p in P.ALL_PINS if p.__name__ in SLOW_PINS])


def _apply(src, edits):
    for old, new in edits:
        n = src.count(old)
        assert n == 1, f"mutation anchor found {n} times: {old!r}"
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    with open(SRC) as f:
        src = _apply(f.read(), edits)
    c = tmp_path / "mutant.c"
    c.write_text(src)
    lib = obuild.build(src=str(c), out=str(tmp_path / "libmutant.so"))
    o = oracle.Oracle(lib)
    failures = []
    for pin in PIN_ORDER:
        try:
            pin(o)
        except AssertionError:
            failures.append(pin.__name__)
            break
        except (ValueError, IndexError, OverflowError):
            failures.append(pin.__name__ + " (error)")
            break
    assert failures, f"no pin caught the mutant '{name}'"
