/* validate_check.c -- every argument check of include/qr.h from plain C, with
 * no GPU work: each call is rejected on the host (n == 0 included), or
 * passes the checks and reaches a launch function that the test program
 * replaces with a stand-in (launch_stubs.cpp), so the pointers below are addresses
 * that are never dereferenced.  Built against a host-sanitized (AddressSanitizer and
 * UndefinedBehaviorSanitizer) build of the C ABI.  Prints one line per
 * failure and "all checks passed" at the end; exit status 0 when every
 * status is the documented one. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qr.h"

static int failures = 0;

#define EXPECT(call, want)                                                          \
  do {                                                                              \
    int got_ = (int)(call);                                                         \
    if (got_ != (int)(want)) {                                                      \
      printf("FAIL line %d: %s -> %d, expected %d\n", __LINE__, #call, got_, (int)(want)); \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

#define P(a) ((void *)(uintptr_t)(a))
#define CP(a) ((const void *)(uintptr_t)(a))

/* Aligned, well-separated addresses (never dereferenced). */
enum { A = 0x10000000, B = 0x20000000, C = 0x30000000, D = 0x40000000 };

static const qr_format kFormats[6] = {QR_INT3, QR_INT4, QR_INT8, QR_ASYM4, QR_ASYM8, QR_FP4};
static const size_t kTile[6] = {896, 1152, 2176, 1072, 2096, 1152};

static void packed_bytes(void) {
  const size_t max_tiles = QR_MAX_TILES;
  for (int f = 0; f < 6; ++f) {
    EXPECT(qr_packed_bytes(kFormats[f], 0), 0);
    EXPECT(qr_packed_bytes(kFormats[f], 2048), kTile[f]);
    EXPECT(qr_packed_bytes(kFormats[f], 3 * 2048), 3 * kTile[f]);
    EXPECT(qr_packed_bytes(kFormats[f], 2047), 0);
    EXPECT(qr_packed_bytes(kFormats[f], 2048 + 1), 0);
    if (qr_packed_bytes(kFormats[f], max_tiles * 2048) != max_tiles * kTile[f]) {
      printf("FAIL: largest tile count, format %d\n", (int)kFormats[f]);
      ++failures;
    }
    EXPECT(qr_packed_bytes(kFormats[f], (max_tiles + 1) * 2048), 0);
    EXPECT(qr_packed_bytes(kFormats[f], SIZE_MAX - SIZE_MAX % 2048), 0);
  }
  EXPECT(qr_packed_bytes((qr_format)0, 2048), 0);
  EXPECT(qr_packed_bytes((qr_format)5, 2048), 0);
  EXPECT(qr_packed_bytes((qr_format)16, 2048), 0);
  EXPECT(qr_packed_bytes((qr_format)32, 2048), 0);
}

static void encode_decode(void) {
  const size_t n = 4 * 2048, huge = ((size_t)QR_MAX_TILES + 1) * 2048;
  for (int f = 0; f < 6; ++f) {
    const qr_format fmt = kFormats[f];
    const size_t pb = 4 * kTile[f];
    /* format / dtype, then sizes, pointers, alignment, aliasing */
    EXPECT(qr_encode(fmt, (qr_dtype)2, CP(A), P(B), n, NULL), QR_ERR_UNSUPPORTED);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A), P(B), n - 1, NULL), QR_ERR_SIZE);
    EXPECT(qr_encode(fmt, QR_BF16, CP(A), P(B), huge, NULL), QR_ERR_SIZE);
    EXPECT(qr_encode(fmt, QR_FP16, NULL, P(B), n, NULL), QR_ERR_ARG);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A), NULL, n, NULL), QR_ERR_ARG);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A + 8), P(B), n, NULL), QR_ERR_ALIGN);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A), P(B + 4), n, NULL), QR_ERR_ALIGN);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A), P(A + 2 * n - 16), n, NULL), QR_ERR_ALIAS);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A + pb - 16), P(A), n, NULL), QR_ERR_ALIAS);
    EXPECT(qr_encode(fmt, QR_FP16, NULL, NULL, 0, NULL), QR_ERR_SIZE);
    EXPECT(qr_encode(fmt, QR_FP16, CP(A), P(B), 0, NULL), QR_ERR_SIZE);
    EXPECT(qr_decode(fmt, (qr_dtype)-1, CP(A), P(B), n, NULL), QR_ERR_UNSUPPORTED);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A), P(B), 100, NULL), QR_ERR_SIZE);
    EXPECT(qr_decode(fmt, QR_BF16, CP(A), P(B), huge, NULL), QR_ERR_SIZE);
    EXPECT(qr_decode(fmt, QR_FP16, NULL, P(B), n, NULL), QR_ERR_ARG);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A), NULL, n, NULL), QR_ERR_ARG);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A + 2), P(B), n, NULL), QR_ERR_ALIGN);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A), P(B + 8), n, NULL), QR_ERR_ALIGN);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A), P(A + pb - 16), n, NULL), QR_ERR_ALIAS);
    EXPECT(qr_decode(fmt, QR_FP16, NULL, NULL, 0, NULL), QR_ERR_SIZE);
    EXPECT(qr_decode(fmt, QR_FP16, CP(A), P(B), 0, NULL), QR_ERR_SIZE);
  }
  EXPECT(qr_encode((qr_format)7, QR_FP16, CP(A), P(B), 2048, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_decode((qr_format)0, QR_FP16, CP(A), P(B), 2048, NULL), QR_ERR_UNSUPPORTED);
}

static void reduce(void) {
  const size_t n = 2048, huge = ((size_t)QR_MAX_TILES + 1) * 2048;
  const void *ranks[QR_MAX_RANKS + 1];
  for (int r = 0; r <= QR_MAX_RANKS; ++r) ranks[r] = CP(A + (uintptr_t)r * 0x100000);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 0, P(B), P(C), n, NULL), QR_ERR_ARG);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, QR_MAX_RANKS + 1, P(B), P(C), n, NULL), QR_ERR_ARG);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(C), n + 2, NULL), QR_ERR_SIZE);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(C), huge, NULL), QR_ERR_SIZE);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, NULL, 2, P(B), P(C), n, NULL), QR_ERR_ARG);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, NULL, P(C), n, NULL), QR_ERR_ARG);
  {
    const void *with_null[2] = {CP(A), NULL};
    EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, with_null, 2, P(B), P(C), n, NULL), QR_ERR_ARG);
    const void *misaligned[2] = {CP(A), CP(A + 0x100000 + 4)};
    EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, misaligned, 2, P(B), P(C), n, NULL), QR_ERR_ALIGN);
  }
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B + 8), P(C), n, NULL), QR_ERR_ALIGN);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(C + 2), n, NULL), QR_ERR_ALIGN);
  /* outputs overlapping a rank, or each other */
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(A + 512), P(C), n, NULL), QR_ERR_ALIAS);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(A + 0x100000 - 1024), n, NULL), QR_ERR_ALIAS);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(B + 1024), n, NULL), QR_ERR_ALIAS);
  /* n == 0 is a size error, checked before the pointers */
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 16, NULL, NULL, 0, NULL), QR_ERR_SIZE);
  EXPECT(qr_reduce_compressed(QR_INT4, QR_FP16, ranks, 2, P(B), P(C), 0, NULL), QR_ERR_SIZE);
  /* formats: unknown, or mixed across the families */
  EXPECT(qr_reduce_compressed((qr_format)5, QR_FP16, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_reduce_compressed(QR_INT4, (qr_dtype)3, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_reduce_compressed_mixed(QR_INT4, QR_ASYM8, QR_FP16, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_reduce_compressed_mixed(QR_ASYM4, QR_INT8, QR_FP16, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_reduce_compressed_mixed(QR_FP4, QR_INT4, QR_FP16, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  EXPECT(qr_reduce_compressed_mixed(QR_INT4, QR_FP4, QR_FP16, ranks, 2, P(B), P(C), n, NULL), QR_ERR_UNSUPPORTED);
  /* the mixed call sizes its output by the output format (2176 B per INT8 tile) */
  EXPECT(qr_reduce_compressed_mixed(QR_INT3, QR_INT8, QR_FP16, ranks, 1, P(A - 1024), NULL, n, NULL), QR_ERR_ALIAS);
  EXPECT(qr_reduce_compressed_mixed(QR_INT4, QR_INT8, QR_BF16, ranks, 1, P(D), NULL, 0, NULL), QR_ERR_SIZE);
}

/* Calls that pass every check reach the launch, which in the test program is
 * a stand-in returning QR_ERR_HIP: the checks do not reject valid calls,
 * including buffers that touch without overlapping and repeated rank buffers. */
static void accepted(void) {
  const size_t n = 4 * 2048;
  const void *ranks[QR_MAX_RANKS];
  for (int r = 0; r < QR_MAX_RANKS; ++r) ranks[r] = CP(A + (uintptr_t)r * 0x100000);
  const void *same[3] = {CP(A), CP(A), CP(A)};
  EXPECT(qr_encode(QR_ASYM4, QR_FP16, CP(A), P(A + 2 * n), n, NULL), QR_ERR_HIP);
  EXPECT(qr_encode(QR_FP4, QR_BF16, CP(A + 4 * 1152), P(A), n, NULL), QR_ERR_HIP);
  EXPECT(qr_decode(QR_ASYM8, QR_FP16, CP(A), P(A + 4 * 2096), n, NULL), QR_ERR_HIP);
  EXPECT(qr_decode(QR_FP4, QR_BF16, CP(A), P(B), n, NULL), QR_ERR_HIP);
  EXPECT(qr_reduce_compressed_mixed(QR_INT3, QR_INT8, QR_FP16, ranks, 1, P(A + 896), NULL, 2048, NULL), QR_ERR_HIP);
  /* an INT3 output (896 B) that ends where the INT4 input starts */
  EXPECT(qr_reduce_compressed_mixed(QR_INT4, QR_INT3, QR_FP16, ranks, 1, P(A - 896), NULL, 2048, NULL), QR_ERR_HIP);
  EXPECT(qr_reduce_compressed(QR_ASYM8, QR_FP16, ranks, QR_MAX_RANKS, P(B), P(C), n, NULL), QR_ERR_HIP);
  EXPECT(qr_reduce_compressed(QR_FP4, QR_BF16, same, 3, P(B), NULL, n, NULL), QR_ERR_HIP);
  EXPECT(qr_reduce_compressed_mixed(QR_ASYM8, QR_ASYM4, QR_BF16, ranks, 2, P(B), P(B + 4 * 1072), n, NULL),
         QR_ERR_HIP);
}

static void status_strings(void) {
  for (int s = 0; s <= 7; ++s) {
    const char *t = qr_status_string((qr_status)s);
    if (!t || !t[0]) {
      printf("FAIL: empty status string %d\n", s);
      ++failures;
    }
  }
  if (strcmp(qr_status_string(QR_OK), "ok") != 0) {
    printf("FAIL: status string of QR_OK\n");
    ++failures;
  }
}

int main(void) {
  packed_bytes();
  encode_decode();
  reduce();
  accepted();
  status_strings();
  if (failures) {
    printf("%d checks failed\n", failures);
    return 1;
  }
  printf("all checks passed\n");
  return 0;
}
