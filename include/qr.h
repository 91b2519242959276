/*
 * qr.h -- C ABI of the MI355X (gfx950) block-quantization codec and the
 * compressed-domain reduction.
 *
 * The method: the send side of a quantized all-reduce encodes its buffer, the
 * reduction runs on the encoded data, and the receive side decodes the result
 * ("QuickReduce INT3 quantization and benchmarking on MI355", introduction and
 * section "Quantization and Dequantization Paths"; the "Flash Communication"
 * review of arXiv 2412.04964, field key_machinery).  This library provides the
 * three steps as single-GPU calls over buffers resident in device memory:
 * qr_encode (send-side quantization), qr_reduce_compressed (decode R encoded
 * buffers, sum, re-encode, decode; qr_reduce_compressed_mixed with separate
 * input and output formats) and qr_decode (receive-side dequantization).
 *
 * Packed format (one per-rank tile per 2048 values, tiles concatenated):
 *   block  = 32 consecutive values sharing one fp16 scale ("Design Highlights")
 *   unit   = 8 consecutive values (value j of a unit is its j-th value)
 *   code   = k + Q with k = clamp(round_half_even(x * e), -Q, Q - 1),
 *            Q = 2^(bits-1): [-4,+3] -> [0,7] for INT3, [-8,+7] -> [0,15] for
 *            INT4, [-128,+127] -> [0,255] for INT8
 *   scale  d = fp16_RNE(min(max|x| / Q, 65504)); e = fp32 1/d (0 if d == 0)
 *   INT4 tile (1152 B): 256 little-endian uint32 words, word u = unit u, value j
 *            at bits 4j..4j+3; then 64 fp16 scales (block g at byte 1024 + 2g)
 *   INT3 tile (896 B):  256 little-endian uint16 words of low code bits (value j
 *            at bits 2j..2j+1), 256 bytes of high code bits (value j at bit j),
 *            then 64 fp16 scales at byte 768 + 2g
 *   INT8 tile (2176 B): 2048 code bytes, then 64 fp16 scales at byte 2048 + 2g
 *   decode: y = (code - Q) * d, exact in fp32, rounded to the I/O dtype.
 *
 * Asymmetric group formats (the "Flash Communication" review of arXiv
 * 2412.04964: fields pith_summary and key_machinery give asymmetric
 * quantization with a scale and a zero point per group of 128; minor_comments
 * on its Algorithm 1 give the dequantization (q - z) * s):
 *   group  = 128 consecutive values, range [lo, hi] = [min(x, 0), max(x, 0)]
 *   scale  s = fp16_RNE(min(fp32 (hi - lo) / (2^b - 1), 65504)),
 *          e = fp32 1/s (0 if s == 0)
 *   zero   z = clamp(round_half_even(-lo * e), 0, 2^b - 1)
 *   code   q = clamp(round_half_even(x * e) + z, 0, 2^b - 1)
 *   QR_ASYM4 tile (1072 B): 1024 B of 4-bit codes laid out as INT4, then 16
 *            fp16 scales (group g at byte 1024 + 2g), then 16 uint8 zero
 *            points (group g at byte 1056 + g)
 *   QR_ASYM8 tile (2096 B): 2048 code bytes, 16 fp16 scales at 2048 + 2g,
 *            16 zero points at 2080 + g
 *   decode: y = (q - z) * s, exact in fp32, rounded to the I/O dtype.  A
 *          zero point above 2^b - 1 is outside the format (the encoder never
 *          writes one); decoding it gives unspecified values.
 *
 * FP4 block format (QR_FP4; "QuickReduce INT3 quantization and benchmarking
 * on MI355", introduction: a hardware-accelerated FP4 path on MI355 that is
 * interchangeable with INT4; the element is OCP MX FP4 E2M1: sign, two
 * exponent bits with bias 1, one mantissa bit, magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6, no inf or NaN):
 *   block  = 32 consecutive values, one fp16 scale d = fp16_RNE(min(m / 6, 65504))
 *            (m = max|x|, so the block maximum maps to 6); e = fp32 1/d (0 if d == 0)
 *   code   = the E2M1 value nearest to fp32(x * e), ties to an even mantissa,
 *            magnitudes above 6 saturating to 6, the sign kept (code 8 = -0)
 *   tile (1152 B): as INT4 -- 256 words of eight 4-bit codes (value j at bits
 *            4j), then 64 fp16 scales at byte 1024 + 2g
 *   decode: y = value(code) * d, exact in fp32, rounded to the I/O dtype.
 *
 * Conventions for every call:
 *   - `n` counts values and must be a positive multiple of 2048, of at most
 *     QR_MAX_TILES = 2^30 tiles; any other n, 0 included, returns QR_ERR_SIZE
 *     (the tile is the unit of the format, and an empty call is a caller error).
 *   - Buffer pointers are DEVICE pointers (hipMalloc or the PyTorch caching
 *     allocator), 16-byte aligned (QR_ERR_ALIGN), owned by the caller.  The
 *     library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream).  Calls only enqueue work and return; the caller synchronizes.
 *   - Arguments are validated on the host before any HIP call, in the order:
 *     format/dtype (QR_ERR_UNSUPPORTED), counts (QR_ERR_ARG / QR_ERR_SIZE),
 *     null pointers (QR_ERR_ARG), alignment (QR_ERR_ALIGN), aliasing
 *     (QR_ERR_ALIAS).  A launch that the HIP runtime refuses returns
 *     QR_ERR_HIP; the status is that of the call's own launch, so an error
 *     left on the thread by an earlier, unrelated HIP call does not fail it.
 *   - Inputs are finite values; NaN/Inf inputs give unspecified codes.
 */
#ifndef QR_H_
#define QR_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below get int as their fixed underlying type, so that any
 * int a C caller passes (an unknown format, say) is a value of the enum and
 * the library's check can reject it without undefined behaviour; in C they
 * are plain enums, passed as int-sized values either way. */
#ifdef __cplusplus
#define QR_ENUM_INT : int
#else
#define QR_ENUM_INT
#endif

typedef enum QR_ENUM_INT {
  QR_OK = 0,
  QR_ERR_ARG = 1,         /* null pointer, R out of [1, QR_MAX_RANKS] */
  QR_ERR_SIZE = 2,        /* n not a multiple of 2048, or more than QR_MAX_TILES tiles */
  QR_ERR_ALIGN = 3,       /* a buffer pointer is not 16-byte aligned */
  QR_ERR_UNSUPPORTED = 4, /* unknown format or dtype */
  QR_ERR_ALIAS = 5,       /* an output overlaps an input or the other output */
  QR_ERR_HIP = 6          /* the HIP runtime refused the kernel launch */
} qr_status;

/* Symmetric 32-value block formats are named by their code width, the
 * asymmetric 128-value group formats by 16 + code width, the FP4 block
 * format by 32 + code width. */
typedef enum QR_ENUM_INT {
  QR_INT3 = 3,
  QR_INT4 = 4,
  QR_INT8 = 8,
  QR_ASYM4 = 20,
  QR_ASYM8 = 24,
  QR_FP4 = 36
} qr_format;

typedef enum QR_ENUM_INT { QR_FP16 = 0, QR_BF16 = 1 } qr_dtype;

#define QR_TILE_VALUES 2048
#define QR_MAX_RANKS 16
/* Largest tile count of a call (2^30 tiles = 2^41 values, beyond any one
 * GPU's memory). */
#define QR_MAX_TILES 1073741824

/* Bytes of the packed form of n values: n / 2048 tiles of 896 (INT3), 1152
 * (INT4 and FP4), 2176 (INT8), 1072 (ASYM4) or 2096 (ASYM8) bytes.  Returns 0
 * for an unknown format, an n that is not a multiple of 2048, or more than
 * QR_MAX_TILES tiles (the calls' own limit).  Tile sizes:
 * "Design Highlights" (INT4 1152 B, INT3 896 B per 2048-value per-rank tile). */
size_t qr_packed_bytes(qr_format fmt, size_t n);

/* Send path ("Quantization and Dequantization Paths": absmax, scale, clip,
 * round, bias, split into planes, write the block scale).
 *   x       device, n values of `dtype` (fp16 or bf16 bit patterns)
 *   packed  device, qr_packed_bytes(fmt, n) bytes, written
 * `packed` must not overlap `x` (QR_ERR_ALIAS). */
qr_status qr_encode(qr_format fmt, qr_dtype dtype, const void *x, void *packed, size_t n,
                    void *stream);

/* Receive path (same section: recombine the bit planes, remove the bias,
 * multiply by the block scale, round to the I/O dtype).
 *   packed  device, qr_packed_bytes(fmt, n) bytes
 *   y       device, n values of `dtype`, written
 * `y` must not overlap `packed` (QR_ERR_ALIAS). */
qr_status qr_decode(qr_format fmt, qr_dtype dtype, const void *packed, void *y, size_t n,
                    void *stream);

/* Compressed-domain reduction of R encoded rank buffers, the in-segment
 * reduction and re-quantization of the two-shot scheme ("Quantization and
 * Dequantization Paths": Phase-1B sums the decoded segments, Phase-2 gathers
 * the re-quantized sum; "Flash Communication": two quantization round trips).
 * For every value: decode each rank exactly into fp32, sum in rank order
 * s = y_0, s = s + y_r for r = 1..R-1, round s to `dtype`, re-encode that
 * block, and (if y_out != NULL) decode the re-encoded value.
 *   packed_ranks  HOST array of R device pointers, each qr_packed_bytes(fmt, n)
 *                 bytes (the array itself is read before the call returns)
 *   R             number of ranks, 1 <= R <= QR_MAX_RANKS (QR_ERR_ARG)
 *   packed_out    device, qr_packed_bytes(fmt, n) bytes, written: the
 *                 re-encoded sum (the payload of the gather)
 *   y_out         device, n values of `dtype`, written, or NULL to skip the
 *                 final decode
 * Neither output may overlap any input or the other output (QR_ERR_ALIAS);
 * input rank buffers may repeat or overlap each other. */
qr_status qr_reduce_compressed(qr_format fmt, qr_dtype dtype, const void *const *packed_ranks,
                               int R, void *packed_out, void *y_out, size_t n, void *stream);

/* The same reduction with the inputs in fmt_in and the re-encoded sum (and its
 * decode) in fmt_out: mixed formats per phase, the "INT6" configuration of the
 * "Flash Communication" review (fields minor_comments, section 3.2.3, and
 * forward_implications: INT4 for the reduce-scatter inputs, INT8 for the
 * all-gather payload).  Any pair of INT3/INT4/INT8 is accepted, and any pair
 * of ASYM4/ASYM8, and FP4 with FP4; pairs across these families are
 * QR_ERR_UNSUPPORTED.  qr_reduce_compressed(f, ...) is
 * qr_reduce_compressed_mixed(f, f, ...).
 *   packed_ranks  HOST array of R device pointers, qr_packed_bytes(fmt_in, n) each
 *   packed_out    device, qr_packed_bytes(fmt_out, n) bytes, written
 *   y_out         device, n values of `dtype`, written, or NULL
 * Validation and errors as for qr_reduce_compressed (an unknown fmt_in or
 * fmt_out is QR_ERR_UNSUPPORTED). */
qr_status qr_reduce_compressed_mixed(qr_format fmt_in, qr_format fmt_out, qr_dtype dtype,
                                     const void *const *packed_ranks, int R, void *packed_out,
                                     void *y_out, size_t n, void *stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char *qr_status_string(qr_status s);

#ifdef __cplusplus
}
#endif

#endif /* QR_H_ */
