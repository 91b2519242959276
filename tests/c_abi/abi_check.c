/* abi_check.c -- the C ABI of include/qr.h used from plain C (no C++, no
 * PyTorch): device memory from the HIP runtime's C API, then encode / decode /
 * reduce calls on values whose results are known exactly.
 *
 * For each symmetric format b and dtype: blocks hold k * s (|k| <= Q, one
 * value of each block at -Q * s) with s a power of two, so encode -> decode
 * returns the input bit for bit, and the reduction of two copies returns 2x
 * bit for bit (the sum 2k * s re-encodes with scale 2s and the same codes).
 * Also: rejected arguments return their documented status without a launch.
 * Prints one line per case; exit status 0 when every check holds. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qr.h"

#define N (4 * QR_TILE_VALUES)

static int failures = 0;

#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      printf("FAIL: " __VA_ARGS__);      \
      printf("\n");                      \
      ++failures;                        \
    }                                    \
  } while (0)

/* fp16 / bf16 bit patterns of k * 2^e for small integers k (exact in both). */
static uint16_t f16_bits(int k, int e) {
  if (k == 0) return 0;
  uint16_t sign = k < 0 ? 0x8000 : 0;
  unsigned m = (unsigned)(k < 0 ? -k : k);
  int p = 0;
  while ((m >> p) > 1) ++p; /* m = 1.f * 2^p */
  unsigned frac = (m << (10 - p)) & 0x3ff;
  return (uint16_t)(sign | ((unsigned)(p + e + 15) << 10) | frac);
}
static uint16_t bf16_bits(int k, int e) {
  if (k == 0) return 0;
  uint16_t sign = k < 0 ? 0x8000 : 0;
  unsigned m = (unsigned)(k < 0 ? -k : k);
  int p = 0;
  while ((m >> p) > 1) ++p;
  unsigned frac = (m << (7 - p)) & 0x7f;
  return (uint16_t)(sign | ((unsigned)(p + e + 127) << 7) | frac);
}

int main(void) {
  const qr_format fmts[3] = {QR_INT3, QR_INT4, QR_INT8};
  const int qs[3] = {4, 8, 128};
  uint16_t *host = (uint16_t *)malloc(N * 2), *back = (uint16_t *)malloc(N * 2), *twice = (uint16_t *)malloc(N * 2);
  void *x, *p0, *out, *y;
  if (hipMalloc(&x, N * 2) != hipSuccess || hipMalloc(&p0, 2176 * 4) != hipSuccess ||
      hipMalloc(&out, 2176 * 4) != hipSuccess || hipMalloc(&y, N * 2) != hipSuccess) {
    printf("FAIL: hipMalloc\n");
    return 1;
  }
  for (int f = 0; f < 3; ++f) {
    for (int dt = 0; dt < 2; ++dt) {
      const int Q = qs[f], e = -3;
      for (int i = 0; i < N; ++i) {
        int k = (i % 32 == 0) ? -Q : ((i * 7919) % (2 * Q)) - Q; /* k in [-Q, Q-1] */
        if (Q == 128) k = (k / 4) * 4;                          /* 2k stays exact in bf16 */
        host[i] = dt == QR_FP16 ? f16_bits(k, e) : bf16_bits(k, e);
        twice[i] = dt == QR_FP16 ? f16_bits(k, e + 1) : bf16_bits(k, e + 1);
      }
      hipMemcpy(x, host, N * 2, hipMemcpyHostToDevice);
      qr_status s = qr_encode(fmts[f], (qr_dtype)dt, x, p0, N, NULL);
      CHECK(s == QR_OK, "encode fmt %d dtype %d: %s", fmts[f], dt, qr_status_string(s));
      s = qr_decode(fmts[f], (qr_dtype)dt, p0, y, N, NULL);
      CHECK(s == QR_OK, "decode fmt %d dtype %d: %s", fmts[f], dt, qr_status_string(s));
      hipDeviceSynchronize();
      hipMemcpy(back, y, N * 2, hipMemcpyDeviceToHost);
      CHECK(memcmp(back, host, N * 2) == 0, "round trip fmt %d dtype %d differs", fmts[f], dt);
      const void *ranks[2] = {p0, p0};
      s = qr_reduce_compressed(fmts[f], (qr_dtype)dt, ranks, 2, out, y, N, NULL);
      CHECK(s == QR_OK, "reduce fmt %d dtype %d: %s", fmts[f], dt, qr_status_string(s));
      hipDeviceSynchronize();
      hipMemcpy(back, y, N * 2, hipMemcpyDeviceToHost);
      CHECK(memcmp(back, twice, N * 2) == 0, "reduce of two copies fmt %d dtype %d is not 2x", fmts[f], dt);
      printf("fmt %d dtype %d: round trip and 2x reduce checked\n", fmts[f], dt);
    }
  }
  /* rejected arguments: no launch, documented status */
  CHECK(qr_encode(QR_INT4, QR_FP16, x, p0, N + 1, NULL) == QR_ERR_SIZE, "size");
  CHECK(qr_encode(QR_INT4, QR_FP16, (char *)x + 2, p0, N, NULL) == QR_ERR_ALIGN, "align");
  CHECK(qr_encode(QR_INT4, QR_FP16, x, x, N, NULL) == QR_ERR_ALIAS, "alias");
  CHECK(qr_encode((qr_format)5, QR_FP16, x, p0, N, NULL) == QR_ERR_UNSUPPORTED, "format");
  CHECK(qr_packed_bytes(QR_FP4, N) == 4 * 1152, "packed bytes");
  CHECK(strcmp(qr_status_string(QR_OK), "ok") == 0, "status string");
  hipFree(x); hipFree(p0); hipFree(out); hipFree(y);
  free(host); free(back); free(twice);
  if (failures) {
    printf("abi_check: %d failures\n", failures);
    return 1;
  }
  printf("abi_check: all checks hold\n");
  return 0;
}
