// qr_api.hip -- the C ABI declared in include/qr.h: host-side argument
// checks (no HIP call before they pass), then the kernel launches of
// qr_kernels.hpp on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "qr.h"
#include "qr_kernels.hpp"

namespace qr {

// ---------------------------------------------------------------------------
// host-side argument checks (no HIP call)
// ---------------------------------------------------------------------------

inline int tile_bytes(int fmt) {
  switch (fmt) {
    case QR_INT3: return Format<3>::kTileBytes;
    case QR_INT4: return Format<4>::kTileBytes;
    case QR_INT8: return Format<8>::kTileBytes;
    case QR_ASYM4: return Format<20>::kTileBytes;
    case QR_ASYM8: return Format<24>::kTileBytes;
    case QR_FP4: return Format<36>::kTileBytes;
    default: return 0;
  }
}

inline bool is_asym(int fmt) { return fmt == QR_ASYM4 || fmt == QR_ASYM8; }

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// The kernels index tiles with an int and advance it by the grid stride (at
// most kMaxGroups * kWavesPerGroup tiles) past the last tile: the tile limit
// leaves room for that step.
static_assert((long long)QR_MAX_TILES + (long long)kMaxGroups * kWavesPerGroup <= 0x7fffffffLL,
              "a tile index plus one grid stride must fit in an int");
inline bool too_large(size_t n) { return n / kTileValues > (size_t)QR_MAX_TILES; }

int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];  // 0 = not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
  if (dev < kMaxDevices) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace qr

using namespace qr;

extern "C" {

size_t qr_packed_bytes(qr_format fmt, size_t n) {
  const int tb = tile_bytes(fmt);
  if (!tb || n % kTileValues || too_large(n)) return 0;
  return n / kTileValues * (size_t)tb;
}

qr_status qr_encode(qr_format fmt, qr_dtype dtype, const void* x, void* packed, size_t n, void* stream) {
  if (!tile_bytes(fmt) || (dtype != QR_FP16 && dtype != QR_BF16)) return QR_ERR_UNSUPPORTED;
  if (n == 0 || n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (!x || !packed) return QR_ERR_ARG;
  if (!aligned16(x) || !aligned16(packed)) return QR_ERR_ALIGN;
  const size_t pb = qr_packed_bytes(fmt, n);
  if (overlap(x, 2 * n, packed, pb)) return QR_ERR_ALIAS;
  const size_t nt = n / kTileValues;
  hipStream_t st = (hipStream_t)stream;
  switch (fmt) {
    case QR_ASYM4:
    case QR_ASYM8: return launch_encode_asym(fmt, dtype, x, packed, nt, st);
    case QR_FP4: return launch_encode_fp4(dtype, x, packed, nt, st);
    case QR_INT3: return launch_encode<3>(dtype, x, packed, nt, st);
    case QR_INT4: return launch_encode<4>(dtype, x, packed, nt, st);
    default: return launch_encode<8>(dtype, x, packed, nt, st);
  }
}

qr_status qr_decode(qr_format fmt, qr_dtype dtype, const void* packed, void* y, size_t n, void* stream) {
  if (!tile_bytes(fmt) || (dtype != QR_FP16 && dtype != QR_BF16)) return QR_ERR_UNSUPPORTED;
  if (n == 0 || n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (!packed || !y) return QR_ERR_ARG;
  if (!aligned16(packed) || !aligned16(y)) return QR_ERR_ALIGN;
  const size_t pb = qr_packed_bytes(fmt, n);
  if (overlap(y, 2 * n, packed, pb)) return QR_ERR_ALIAS;
  const size_t nt = n / kTileValues;
  hipStream_t st = (hipStream_t)stream;
  switch (fmt) {
    case QR_ASYM4:
    case QR_ASYM8: return launch_decode_asym(fmt, dtype, packed, y, nt, st);
    case QR_FP4: return launch_decode_fp4(dtype, packed, y, nt, st);
    case QR_INT3: return launch_decode<3>(dtype, packed, y, nt, st);
    case QR_INT4: return launch_decode<4>(dtype, packed, y, nt, st);
    default: return launch_decode<8>(dtype, packed, y, nt, st);
  }
}

qr_status qr_reduce_compressed_mixed(qr_format fmt_in, qr_format fmt_out, qr_dtype dtype,
                                     const void* const* packed_ranks, int R, void* packed_out, void* y_out,
                                     size_t n, void* stream) {
  if (!tile_bytes(fmt_in) || !tile_bytes(fmt_out) || (dtype != QR_FP16 && dtype != QR_BF16) ||
      is_asym(fmt_in) != is_asym(fmt_out) || (fmt_in == QR_FP4) != (fmt_out == QR_FP4))
    return QR_ERR_UNSUPPORTED;
  if (R < 1 || R > QR_MAX_RANKS) return QR_ERR_ARG;
  if (n == 0 || n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (!packed_ranks || !packed_out) return QR_ERR_ARG;
  for (int r = 0; r < R; ++r)
    if (!packed_ranks[r]) return QR_ERR_ARG;
  for (int r = 0; r < R; ++r)
    if (!aligned16(packed_ranks[r])) return QR_ERR_ALIGN;
  if (!aligned16(packed_out) || (y_out && !aligned16(y_out))) return QR_ERR_ALIGN;
  const size_t pin = qr_packed_bytes(fmt_in, n), pout = qr_packed_bytes(fmt_out, n);
  for (int r = 0; r < R; ++r) {
    if (overlap(packed_ranks[r], pin, packed_out, pout)) return QR_ERR_ALIAS;
    if (y_out && overlap(packed_ranks[r], pin, y_out, 2 * n)) return QR_ERR_ALIAS;
  }
  if (y_out && overlap(packed_out, pout, y_out, 2 * n)) return QR_ERR_ALIAS;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int r = 0; r < R; ++r) a.ranks[r] = (const uint8_t*)packed_ranks[r];
  a.out = (uint8_t*)packed_out;
  a.y = (uint8_t*)y_out;
  a.R = R;
  a.ntiles = (int)(n / kTileValues);
  hipStream_t st = (hipStream_t)stream;
  if (fmt_in == QR_ASYM4) return launch_reduce_asym_from20(fmt_out, dtype, a, st);
  if (fmt_in == QR_ASYM8) return launch_reduce_asym_from24(fmt_out, dtype, a, st);
  if (fmt_in == QR_FP4) return launch_reduce_fp4(dtype, a, st);
  if (fmt_in != fmt_out) {
    switch (fmt_in) {
      case QR_INT3: return launch_reduce_mixed_from3(fmt_out, dtype, a, st);
      case QR_INT4: return launch_reduce_mixed_from4(fmt_out, dtype, a, st);
      default: return launch_reduce_mixed_from8(fmt_out, dtype, a, st);
    }
  }
  switch (fmt_in) {
    case QR_INT3: return launch_reduce<3, 3>(dtype, a, st);
    case QR_INT4: return launch_reduce<4, 4>(dtype, a, st);
    default: return launch_reduce<8, 8>(dtype, a, st);
  }
}

qr_status qr_reduce_compressed(qr_format fmt, qr_dtype dtype, const void* const* packed_ranks, int R,
                               void* packed_out, void* y_out, size_t n, void* stream) {
  return qr_reduce_compressed_mixed(fmt, fmt, dtype, packed_ranks, R, packed_out, y_out, n, stream);
}

const char* qr_status_string(qr_status s) {
  switch (s) {
    case QR_OK: return "ok";
    case QR_ERR_ARG: return "invalid argument (null pointer or rank count)";
    case QR_ERR_SIZE: return "value count is not a multiple of 2048 or exceeds QR_MAX_TILES (2^30) tiles";
    case QR_ERR_ALIGN: return "buffer pointer is not 16-byte aligned";
    case QR_ERR_UNSUPPORTED: return "unsupported format or dtype";
    case QR_ERR_ALIAS: return "output buffer overlaps another buffer";
    case QR_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"
