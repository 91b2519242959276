/*
 * qr_oracle.c -- plain, slow CPU oracle of the 32-value block codec
 * (INT3 / INT4 / INT8) and of the compressed-domain reduction.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path
 * (the HIP library) never links, loads or calls it, and this file shares no
 * source, header, table or helper with the HIP path.
 *
 * What it follows:
 *  [QR]  "QuickReduce INT3 quantization and benchmarking on MI355" (AMD blog),
 *        section "Design Highlights": a block of 32 FP16/BF16 values shares
 *        one FP16 scale; values are scaled, clipped to the symmetric signed
 *        range, rounded and biased to unsigned codes; INT4 holds eight 4-bit
 *        codes in one 32-bit word; INT3 puts the low two bits of eight codes
 *        in one uint16 and the high bit of eight codes in one uint8; a
 *        2048-value per-rank tile is 1152 bytes for INT4 and 896 bytes for
 *        INT3.
 *  [QR-Q] same page, section "Quantization and Dequantization Paths": the
 *        send path takes the block absolute maximum, derives the scale,
 *        scales / clips / rounds / biases, splits and stores the planes and
 *        the scale; the receive path recombines the bits, removes the bias
 *        and multiplies by the scale; the two-shot kernel sums the decoded
 *        segments, then re-quantizes the sum for the gather.
 *  [FC]  "Flash Communication" review (arXiv 2412.04964), fields
 *        key_machinery / core_discovery: only two quantization round trips
 *        (quantize, exchange, decode + local sum, re-quantize, gather,
 *        decode).
 *  [NIB] vLLM PR #54965 description (nibble n%8 of a packed int32 word at
 *        bits 4*(n%8)) and vLLM PR #43389 (GPTQ sequential shifts
 *        0,4,...,28): value j of a word sits at the lowest bits first.
 *
 * Readings taken where the pages are silent (each one is named where it is
 * used below):
 *  R1  block = 32 contiguous values; one unit = 8 contiguous values
 *      (one INT4 word, one INT3 uint16 + uint8).
 *  R2  scale d = fp16_RNE(min(m / 2^(b-1), 65504)); m / 2^(b-1) is exact.
 *  R3  the encode multiplier is e = fp32_RN(1 / d), or 0 when d == 0; it is
 *      kept in fp32 (a literal fp16 reciprocal overflows for small blocks).
 *  R4  round half to even; clip before rounding, as the page orders it.
 *  R5  tile regions: INT4 [1024 B codes | 128 B scales]; INT3 [512 B 2-bit
 *      plane | 256 B 1-bit plane | 128 B scales]; INT8 [2048 B codes |
 *      128 B scales] (INT8 extends the same framework to b = 8).
 *  R6  the reduction decodes each rank exactly into fp32, sums in fixed rank
 *      order 0..R-1 starting from rank 0's value, rounds the sum to the I/O
 *      dtype, re-encodes it, and decodes that re-encoded tile.
 *  R7  asymmetric group codec ([FC] pith_summary / key_machinery: asymmetric
 *      quantization with group size 128, a scale and a zero point per group;
 *      minor_comments on Algorithm 1: dequantize as (q - z) * s): a group is
 *      128 consecutive values; its range [lo, hi] always includes 0 (lo =
 *      min(min x, 0), hi = max(max x, 0)); s = fp16_RNE(min(RN32(RN32(hi - lo)
 *      / (2^b - 1)), 65504)); e = RN32(1 / s) (0 when s == 0); z =
 *      clamp(rint(RN32(-lo * e)), 0, 2^b - 1); q = clamp(rint(RN32(x * e)) + z,
 *      0, 2^b - 1); decode (q - z) * s, exact in fp32.  A tile of 2048 values
 *      is [codes (as INT4 / INT8) | 16 fp16 scales | 16 uint8 zero points]:
 *      1072 bytes for 4-bit codes, 2096 for 8-bit.
 *  R8  FP4 block codec ([QR] introduction: a hardware-accelerated FP4 path on
 *      MI355 that is interchangeable with INT4; the page gives no format): the
 *      element is OCP MX FP4 E2M1 (bit 3 sign, bits 2..1 exponent with bias 1,
 *      bit 0 mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no inf or NaN),
 *      in INT4's framework: blocks of 32 values with one fp16 scale, codes
 *      packed as INT4 nibbles, a 1152-byte tile [1024 B codes | 128 B scales].
 *      d = fp16_RNE(min(RN32(m / 6), 65504)) (the block maximum maps to the
 *      largest magnitude 6); e = RN32(1 / d) (0 when d == 0); the code of x is
 *      the E2M1 value nearest to RN32(x * e), ties to an even mantissa,
 *      magnitudes above 6 saturating to 6, the sign kept (so a negative value
 *      that rounds to zero is -0, code 8); decode = value * d, exact in fp32.
 *
 * All floating point is IEEE binary32 with round-to-nearest-even; build with
 * -O2 -ffp-contract=off and without -ffast-math.  binary32, not binary64:
 * floating point here decides integers (codes, scales, zero points, the
 * re-quantized sum), and those decisions are taken in the GPU kernels'
 * precision; every decoded value and product is exact in binary32.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define QRO_TILE 2048  /* values per per-rank tile [QR] */
#define QRO_BLOCK 32   /* values per shared scale [QR] */
#define QRO_BLOCKS (QRO_TILE / QRO_BLOCK)

enum { QRO_FP16 = 0, QRO_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* binary16 and bfloat16 conversions, from the IEEE 754 format definitions   */
/* ------------------------------------------------------------------------ */

/* binary16: sign, 5 exponent bits with bias 15, 10 fraction bits. */
float qro_f16_to_f32(uint16_t h) {
  int sign = h >> 15;
  int exp = (h >> 10) & 31;
  int frac = h & 1023;
  float mag;
  if (exp == 0)
    mag = ldexpf((float)frac, -24); /* subnormal: frac * 2^-24 */
  else if (exp == 31)
    mag = frac ? NAN : INFINITY;
  else
    mag = ldexpf((float)(1024 + frac), exp - 25); /* (1024+frac) * 2^(exp-15-10) */
  return sign ? -mag : mag;
}

/* Nearest binary16 value, ties to the even fraction. */
uint16_t qro_f32_to_f16(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  float a = fabsf(x);
  if (isnan(a)) return sign | 0x7e00;
  /* 65520 is the midpoint between the largest finite value 65504 (odd
     fraction) and 2^16: it and everything above rounds to infinity. */
  if (a >= 65520.0f) return sign | 0x7c00;
  float quantum; /* spacing of binary16 values near a */
  if (a < 0x1p-14f) {
    quantum = 0x1p-24f;
  } else {
    int e;
    frexpf(a, &e); /* a in [2^(e-1), 2^e) */
    quantum = ldexpf(1.0f, e - 1 - 10);
  }
  /* a / quantum is exact (power of two); rintf rounds half to even. */
  float r = rintf(a / quantum) * quantum;
  if (r < 0x1p-14f) return sign | (uint16_t)(r / 0x1p-24f);
  int e;
  frexpf(r, &e);
  int E = e - 1; /* r in [2^E, 2^(E+1)) */
  uint16_t frac = (uint16_t)(r / ldexpf(1.0f, E - 10) - 1024.0f);
  return sign | (uint16_t)((E + 15) << 10) | frac;
}

/* bfloat16 is the upper half of a binary32 pattern. */
float qro_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Nearest bfloat16 value (8 significant bits), ties to even. */
uint16_t qro_f32_to_bf16(float x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  float a = fabsf(x);
  if (isnan(a)) return sign | 0x7fc0;
  /* midpoint between the largest finite value (2 - 2^-7) * 2^127 and 2^128 */
  if (a >= 0x1.ffp127f) return sign | 0x7f80;
  float quantum;
  if (a < 0x1p-126f) {
    quantum = 0x1p-133f;
  } else {
    int e;
    frexpf(a, &e);
    quantum = ldexpf(1.0f, e - 1 - 7);
  }
  float r = rintf(a / quantum) * quantum; /* exact scaling, ties to even */
  uint32_t u;
  memcpy(&u, &r, sizeof u); /* r is a bfloat16 value: its low 16 bits are 0 */
  return sign | (uint16_t)(u >> 16);
}

static float dtype_to_f32(int dtype, uint16_t v) {
  return dtype == QRO_FP16 ? qro_f16_to_f32(v) : qro_bf16_to_f32(v);
}

static uint16_t f32_to_dtype(int dtype, float x) {
  return dtype == QRO_FP16 ? qro_f32_to_f16(x) : qro_f32_to_bf16(x);
}

/* ------------------------------------------------------------------------ */
/* tile layout (R1, R5)                                                      */
/* ------------------------------------------------------------------------ */

/* Format ids: 3, 4, 8 = symmetric block codec with that many bits; 20, 24 =
   asymmetric group codec with 4 or 8 bits (R7); 36 = FP4 E2M1 block codec
   (R8), laid out like INT4. */
#define QRO_ASYM 16
#define QRO_FP4 36
static int fmt_bits(int fmt) {
  if (fmt == 3 || fmt == 4 || fmt == 8) return fmt;
  if (fmt == QRO_ASYM + 4 || fmt == QRO_ASYM + 8) return fmt - QRO_ASYM;
  if (fmt == QRO_FP4) return 4;
  return 0;
}
static int fmt_asym(int fmt) { return fmt == QRO_ASYM + 4 || fmt == QRO_ASYM + 8; }
static int fmt_fp4(int fmt) { return fmt == QRO_FP4; }

#define QRO_AGROUP 128 /* values per asymmetric group (R7) */
#define QRO_AGROUPS (QRO_TILE / QRO_AGROUP)

/* Bytes of one tile: code planes plus 64 binary16 scales. */
static size_t tile_bytes(int bits) {
  size_t code_bits = (size_t)QRO_TILE * (size_t)bits;
  return code_bits / 8 + 2 * QRO_BLOCKS;
}

/* Asymmetric tile: codes plus 16 binary16 scales and 16 uint8 zero points. */
static size_t asym_tile_bytes(int bits) {
  return (size_t)QRO_TILE * (size_t)bits / 8 + 3 * QRO_AGROUPS;
}

static size_t fmt_tile_bytes(int fmt) {
  return fmt_asym(fmt) ? asym_tile_bytes(fmt_bits(fmt)) : tile_bytes(fmt_bits(fmt));
}

/* Byte offset of the scale region inside a tile. */
static size_t scale_offset(int bits) { return (size_t)QRO_TILE * (size_t)bits / 8; }

size_t qro_packed_bytes(int fmt, size_t n) {
  int bits = fmt_bits(fmt);
  if (!bits || n % QRO_TILE) return 0;
  return n / QRO_TILE * fmt_tile_bytes(fmt);
}

/* INT3: the 2-bit plane is 256 little-endian uint16 words (word u holds the
   low two bits of values 8u..8u+7, value j at bits 2j), then the 1-bit plane
   is 256 bytes (byte u holds bit 2 of the same values, value j at bit j). */
#define INT3_Q1_OFFSET 512

static void put_code(int bits, uint8_t *tile, int i, unsigned code) {
  int u = i / 8, j = i % 8;
  if (bits == 3) {
    unsigned w = tile[2 * u] | (tile[2 * u + 1] << 8);
    w |= (code & 3u) << (2 * j);
    tile[2 * u] = (uint8_t)(w & 0xff);
    tile[2 * u + 1] = (uint8_t)(w >> 8);
    tile[INT3_Q1_OFFSET + u] |= (uint8_t)(((code >> 2) & 1u) << j);
  } else if (bits == 4) {
    /* word u little-endian; value j at bits 4j..4j+3 [NIB] */
    uint32_t w = (uint32_t)tile[4 * u] | ((uint32_t)tile[4 * u + 1] << 8) |
                 ((uint32_t)tile[4 * u + 2] << 16) | ((uint32_t)tile[4 * u + 3] << 24);
    w |= (uint32_t)code << (4 * j);
    tile[4 * u] = (uint8_t)w;
    tile[4 * u + 1] = (uint8_t)(w >> 8);
    tile[4 * u + 2] = (uint8_t)(w >> 16);
    tile[4 * u + 3] = (uint8_t)(w >> 24);
  } else {
    tile[i] = (uint8_t)code;
  }
}

static unsigned get_code(int bits, const uint8_t *tile, int i) {
  int u = i / 8, j = i % 8;
  if (bits == 3) {
    unsigned w = tile[2 * u] | (tile[2 * u + 1] << 8);
    unsigned low = (w >> (2 * j)) & 3u;
    unsigned high = (tile[INT3_Q1_OFFSET + u] >> j) & 1u;
    return low | (high << 2);
  } else if (bits == 4) {
    uint32_t w = (uint32_t)tile[4 * u] | ((uint32_t)tile[4 * u + 1] << 8) |
                 ((uint32_t)tile[4 * u + 2] << 16) | ((uint32_t)tile[4 * u + 3] << 24);
    return (w >> (4 * j)) & 15u;
  }
  return tile[i];
}

static uint16_t get_scale(int bits, const uint8_t *tile, int g) {
  const uint8_t *p = tile + scale_offset(bits) + 2 * g;
  return (uint16_t)(p[0] | (p[1] << 8));
}

static void put_scale(int bits, uint8_t *tile, int g, uint16_t d) {
  uint8_t *p = tile + scale_offset(bits) + 2 * g;
  p[0] = (uint8_t)(d & 0xff);
  p[1] = (uint8_t)(d >> 8);
}

/* ------------------------------------------------------------------------ */
/* one block: scale, quantize, dequantize                                    */
/* ------------------------------------------------------------------------ */

/* Scale of a block with absolute maximum m (R2, R3). */
void qro_block_scale(int bits, float m, uint16_t *d_bits, float *e) {
  const int Q = 1 << (bits - 1);
  float t = m / (float)Q;         /* exact: Q is a power of two */
  if (t > 65504.0f) t = 65504.0f; /* largest finite binary16 */
  *d_bits = qro_f32_to_f16(t);
  float d = qro_f16_to_f32(*d_bits);
  *e = (d == 0.0f) ? 0.0f : 1.0f / d;
}

/* Send path of one block [QR-Q]: absmax, scale, scale values, clip to
   [-Q, Q-1], round half to even (R4), bias by Q. */
static void encode_block(int bits, const float x[QRO_BLOCK], unsigned codes[QRO_BLOCK],
                         uint16_t *d_bits) {
  const int Q = 1 << (bits - 1);
  float m = 0.0f;
  for (int i = 0; i < QRO_BLOCK; ++i) {
    float a = fabsf(x[i]);
    if (a > m) m = a;
  }
  float e;
  qro_block_scale(bits, m, d_bits, &e);
  for (int i = 0; i < QRO_BLOCK; ++i) {
    float v = x[i] * e;
    float c = fminf(fmaxf(v, -(float)Q), (float)(Q - 1));
    long k = lrintf(c); /* default rounding mode: to nearest, ties to even */
    codes[i] = (unsigned)(k + Q);
  }
}

/* Receive path of one value [QR-Q]: remove the bias, multiply by the scale.
   (code - Q) has at most 8 significant bits and the scale 11, so the product
   is exact in binary32. */
static float decode_value(int bits, const uint8_t *tile, int i) {
  const int Q = 1 << (bits - 1);
  unsigned code = get_code(bits, tile, i);
  float d = qro_f16_to_f32(get_scale(bits, tile, i / QRO_BLOCK));
  return (float)((int)code - Q) * d;
}

/* Encode one tile of binary32 values that are exactly representable in the
   I/O dtype. */
static void encode_tile(int bits, const float *x, uint8_t *tile) {
  memset(tile, 0, tile_bytes(bits));
  for (int g = 0; g < QRO_BLOCKS; ++g) {
    unsigned codes[QRO_BLOCK];
    uint16_t d_bits;
    encode_block(bits, x + g * QRO_BLOCK, codes, &d_bits);
    for (int i = 0; i < QRO_BLOCK; ++i) put_code(bits, tile, g * QRO_BLOCK + i, codes[i]);
    put_scale(bits, tile, g, d_bits);
  }
}

/* ------------------------------------------------------------------------ */
/* asymmetric group codec (R7)                                              */
/* ------------------------------------------------------------------------ */

static size_t asym_scale_offset(int bits) { return (size_t)QRO_TILE * (size_t)bits / 8; }
static size_t asym_zero_offset(int bits) { return asym_scale_offset(bits) + 2 * QRO_AGROUPS; }

/* Scale, multiplier and zero point of a group with range [lo, hi] (lo <= 0 <= hi). */
void qro_group_params(int bits, float lo, float hi, uint16_t *d_bits, float *e, int *z) {
  const int qmax = (1 << bits) - 1;
  float t = (hi - lo) / (float)qmax;
  if (t > 65504.0f) t = 65504.0f; /* saturate the group scale */
  *d_bits = qro_f32_to_f16(t);
  float d = qro_f16_to_f32(*d_bits);
  *e = (d == 0.0f) ? 0.0f : 1.0f / d; /* group multiplier */
  float zf = rintf(-lo * *e);
  zf = fminf(fmaxf(zf, 0.0f), (float)qmax);
  *z = (int)zf;
}

static void encode_group_asym(int bits, const float x[QRO_AGROUP], unsigned codes[QRO_AGROUP],
                              uint16_t *d_bits, int *z) {
  const int qmax = (1 << bits) - 1;
  float lo = 0.0f, hi = 0.0f; /* the range always includes 0 */
  for (int i = 0; i < QRO_AGROUP; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  float e;
  qro_group_params(bits, lo, hi, d_bits, &e, z);
  for (int i = 0; i < QRO_AGROUP; ++i) {
    float u = x[i] * e;
    /* rint(u) + z in binary32: exact while |u| < 2^24, and an infinite u (a
       sum that overflowed the I/O dtype) stays infinite, so the clamp sends
       it to the end of the range, as the definition does */
    float k = rintf(u) + (float)*z;
    k = fminf(fmaxf(k, 0.0f), (float)qmax);
    codes[i] = (unsigned)k;
  }
}

static void encode_tile_asym(int bits, const float *x, uint8_t *tile) {
  memset(tile, 0, asym_tile_bytes(bits));
  for (int g = 0; g < QRO_AGROUPS; ++g) {
    unsigned codes[QRO_AGROUP];
    uint16_t d_bits;
    int z;
    encode_group_asym(bits, x + g * QRO_AGROUP, codes, &d_bits, &z);
    for (int i = 0; i < QRO_AGROUP; ++i) put_code(bits, tile, g * QRO_AGROUP + i, codes[i]);
    uint8_t *p = tile + asym_scale_offset(bits) + 2 * g;
    p[0] = (uint8_t)(d_bits & 0xff);
    p[1] = (uint8_t)(d_bits >> 8);
    tile[asym_zero_offset(bits) + g] = (uint8_t)z;
  }
}

/* Algorithm 1 of the Flash Communication paper as the review describes it:
   (q - z) * s, exact in fp32 (|q - z| < 2^8, s has 11 significant bits). */
static float decode_value_asym(int bits, const uint8_t *tile, int i) {
  int g = i / QRO_AGROUP;
  const uint8_t *p = tile + asym_scale_offset(bits) + 2 * g;
  float d = qro_f16_to_f32((uint16_t)(p[0] | (p[1] << 8)));
  int z = tile[asym_zero_offset(bits) + g];
  return (float)((int)get_code(bits, tile, i) - z) * d;
}

/* ------------------------------------------------------------------------ */
/* FP4 E2M1 block codec (R8)                                                 */
/* ------------------------------------------------------------------------ */

/* Value of an E2M1 code: exponent field 0 holds 0 and the subnormal 0.5
   (mantissa * 2^-1); fields 1..3 hold (1 + mantissa / 2) * 2^(field - 1). */
static float fp4_value(unsigned code) {
  int ef = (code >> 1) & 3, m = code & 1;
  float mag = ef == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, ef - 1);
  return (code & 8u) ? -mag : mag;
}

/* Code of the E2M1 value nearest to v: round to nearest, ties to even, at the
   spacing of v's binade (0.5 below 2, 1 in [2, 4), 2 from 4 on), then
   saturate magnitudes above 6; the sign bit is v's sign. */
static unsigned fp4_code(float v) {
  float a = fabsf(v);
  float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
  float r = rintf(a / step) * step; /* exact: the step is a power of two */
  if (r > 6.0f) r = 6.0f;
  unsigned mc = 0;
  while (mc < 7 && fp4_value(mc) != r) ++mc; /* r is one of the eight magnitudes */
  return (signbit(v) ? 8u : 0u) | mc;
}

/* Scale of an FP4 block with absolute maximum m: the maximum maps to 6. */
void qro_fp4_block_scale(float m, uint16_t *d_bits, float *e) {
  float t = m / 6.0f;             /* correctly rounded binary32 quotient */
  if (t > 65504.0f) t = 65504.0f; /* saturate at the largest binary16 */
  *d_bits = qro_f32_to_f16(t);
  float d = qro_f16_to_f32(*d_bits);
  *e = (d == 0.0f) ? 0.0f : 1.0f / d; /* FP4 multiplier */
}

static void encode_tile_fp4(const float *x, uint8_t *tile) {
  memset(tile, 0, tile_bytes(4));
  for (int g = 0; g < QRO_BLOCKS; ++g) {
    const float *xb = x + g * QRO_BLOCK;
    float m = 0.0f;
    for (int i = 0; i < QRO_BLOCK; ++i)
      if (fabsf(xb[i]) > m) m = fabsf(xb[i]);
    uint16_t d_bits;
    float e;
    qro_fp4_block_scale(m, &d_bits, &e);
    for (int i = 0; i < QRO_BLOCK; ++i) put_code(4, tile, g * QRO_BLOCK + i, fp4_code(xb[i] * e));
    put_scale(4, tile, g, d_bits);
  }
}

/* value * d is exact in binary32 (2 and 11 significant bits). */
static float decode_value_fp4(const uint8_t *tile, int i) {
  return fp4_value(get_code(4, tile, i)) * qro_f16_to_f32(get_scale(4, tile, i / QRO_BLOCK));
}

/* Format-generic tile encode / value decode. */
static void encode_tile_fmt(int fmt, const float *x, uint8_t *tile) {
  if (fmt_asym(fmt))
    encode_tile_asym(fmt_bits(fmt), x, tile);
  else if (fmt_fp4(fmt))
    encode_tile_fp4(x, tile);
  else
    encode_tile(fmt_bits(fmt), x, tile);
}

static float decode_value_fmt(int fmt, const uint8_t *tile, int i) {
  if (fmt_asym(fmt)) return decode_value_asym(fmt_bits(fmt), tile, i);
  if (fmt_fp4(fmt)) return decode_value_fp4(tile, i);
  return decode_value(fmt_bits(fmt), tile, i);
}

/* ------------------------------------------------------------------------ */
/* exported entry points                                                     */
/* ------------------------------------------------------------------------ */

static int check(int fmt, int dtype, size_t n) {
  if (!fmt_bits(fmt)) return -1;
  if (dtype != QRO_FP16 && dtype != QRO_BF16) return -1;
  if (n % QRO_TILE) return -1;
  return 0;
}

int qro_encode(int fmt, int dtype, const uint16_t *x, uint8_t *packed, size_t n) {
  if (check(fmt, dtype, n)) return -1;
  size_t tb = fmt_tile_bytes(fmt);
  float xf[QRO_TILE];
  for (size_t t = 0; t < n / QRO_TILE; ++t) {
    for (int i = 0; i < QRO_TILE; ++i) xf[i] = dtype_to_f32(dtype, x[t * QRO_TILE + i]);
    encode_tile_fmt(fmt, xf, packed + t * tb);
  }
  return 0;
}

/* Exact binary32 decode (before any rounding to the I/O dtype). */
int qro_decode_f32(int fmt, const uint8_t *packed, float *y, size_t n) {
  if (check(fmt, QRO_FP16, n)) return -1;
  size_t tb = fmt_tile_bytes(fmt);
  for (size_t t = 0; t < n / QRO_TILE; ++t)
    for (int i = 0; i < QRO_TILE; ++i) y[t * QRO_TILE + i] = decode_value_fmt(fmt, packed + t * tb, i);
  return 0;
}

int qro_decode(int fmt, int dtype, const uint8_t *packed, uint16_t *y, size_t n) {
  if (check(fmt, dtype, n)) return -1;
  size_t tb = fmt_tile_bytes(fmt);
  for (size_t t = 0; t < n / QRO_TILE; ++t)
    for (int i = 0; i < QRO_TILE; ++i)
      y[t * QRO_TILE + i] = f32_to_dtype(dtype, decode_value_fmt(fmt, packed + t * tb, i));
  return 0;
}

/* Compressed-domain reduction over R rank buffers (R6, [QR-Q], [FC]), with
   the inputs in format fmt_in and the re-encoded sum in fmt_out.  Mixed
   formats per phase follow the Flash Communication review's "INT6"
   configuration (fields minor_comments, section 3.2.3, and
   forward_implications): 4-bit codes for the reduce-scatter inputs, 8-bit
   codes for the all-gather payload. */
int qro_reduce_mixed(int fmt_in, int fmt_out, int dtype, const uint8_t *const *ranks, int R,
                     uint8_t *packed_out, uint16_t *y_out, size_t n) {
  if (check(fmt_in, dtype, n) || check(fmt_out, dtype, n) || R < 1) return -1;
  size_t tb = fmt_tile_bytes(fmt_in), otb = fmt_tile_bytes(fmt_out);
  float z[QRO_TILE];
  for (size_t t = 0; t < n / QRO_TILE; ++t) {
    for (int i = 0; i < QRO_TILE; ++i) {
      float s = decode_value_fmt(fmt_in, ranks[0] + t * tb, i);
      for (int r = 1; r < R; ++r) s = s + decode_value_fmt(fmt_in, ranks[r] + t * tb, i);
      z[i] = dtype_to_f32(dtype, f32_to_dtype(dtype, s));
    }
    uint8_t *out = packed_out + t * otb;
    encode_tile_fmt(fmt_out, z, out);
    if (y_out)
      for (int i = 0; i < QRO_TILE; ++i)
        y_out[t * QRO_TILE + i] = f32_to_dtype(dtype, decode_value_fmt(fmt_out, out, i));
  }
  return 0;
}

/* The same-format reduction. */
int qro_reduce(int fmt, int dtype, const uint8_t *const *ranks, int R, uint8_t *packed_out,
               uint16_t *y_out, size_t n) {
  return qro_reduce_mixed(fmt, fmt, dtype, ranks, R, packed_out, y_out, n);
}

/* Array forms of the conversions above, for the converter pins. */
void qro_f32_to_f16_array(const float *x, uint16_t *h, size_t n) {
  for (size_t i = 0; i < n; ++i) h[i] = qro_f32_to_f16(x[i]);
}
void qro_f16_to_f32_array(const uint16_t *h, float *x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = qro_f16_to_f32(h[i]);
}
void qro_f32_to_bf16_array(const float *x, uint16_t *b, size_t n) {
  for (size_t i = 0; i < n; ++i) b[i] = qro_f32_to_bf16(x[i]);
}
void qro_bf16_to_f32_array(const uint16_t *b, float *x, size_t n) {
  for (size_t i = 0; i < n; ++i) x[i] = qro_bf16_to_f32(b[i]);
}
