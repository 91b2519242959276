// qr_kernels.hip -- gfx950 kernels and the C ABI declared in include/qr.h.
//
// Three kernels, each with one 64-lane wave per 2048-value tile and one lane
// per 32-value block (the codec itself is in qr_codec.hpp):
//   encode  fp16/bf16 tile -> LDS (row order) -> lane block -> packed tile
//   decode  packed block -> lane -> LDS (block order) -> fp16/bf16 tile
//   reduce  R packed blocks -> exact fp32 decode + rank-order sum -> round to
//           dtype -> re-encode (packed_out) -> decode (y_out, through LDS)
// The reduce is the in-segment reduction + re-quantization of the two-shot
// all-reduce ("QuickReduce INT3 quantization and benchmarking on MI355",
// "Quantization and Dequantization Paths"; "Flash Communication" review,
// key_machinery): two quantization round trips, decode-sum-encode fused so
// that the fp32 sum never leaves registers.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "qr.h"
#include "qr_codec.hpp"

namespace qr {

constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kMaxGroups = 8192;

// ---------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void encode_kernel(const uint8_t* __restrict__ x,
                                                          uint8_t* __restrict__ packed, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kChunks];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  u32x4* tl = lds[wave];
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < ntiles; tile += gridDim.x * kWavesPerGroup) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)tile * (kTileValues * 2));
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(src + lane + kWave * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) tl[swz(lane + kWave * k)] = v[k];
    wave_lds_sync();
    float z[kBlockValues];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 c = tl[swz(4 * lane + j)];
      const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        z[8 * j + 2 * q] = lo_to_f32<DT>(w[q]);
        z[8 * j + 2 * q + 1] = hi_to_f32<DT>(w[q]);
      }
    }
    wave_lds_sync();  // the next tile overwrites this LDS tile
    Block<BITS> blk;
    float k[kBlockValues];
    const uint32_t scale = encode_block<BITS>(z, blk, k);
    store_block<BITS>(packed + (size_t)tile * Format<BITS>::kTileBytes, lane, blk, scale);
  }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// Writes one lane's 32 output values (block order) and stores the wave's
// tile in row order.
template <int DT>
__device__ __forceinline__ void store_tile_values(u32x4* tl, int lane, const float (&y)[kBlockValues],
                                                  uint8_t* __restrict__ dst) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 c;
    c.x = pack2<DT>(y[8 * j + 0], y[8 * j + 1]);
    c.y = pack2<DT>(y[8 * j + 2], y[8 * j + 3]);
    c.z = pack2<DT>(y[8 * j + 4], y[8 * j + 5]);
    c.w = pack2<DT>(y[8 * j + 6], y[8 * j + 7]);
    tl[swz(4 * lane + j)] = c;
  }
  wave_lds_sync();
  u32x4* out = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int k = 0; k < 4; ++k) __builtin_nontemporal_store(tl[swz(lane + kWave * k)], out + lane + kWave * k);
  wave_lds_sync();
}

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ y, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kChunks];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < ntiles; tile += gridDim.x * kWavesPerGroup) {
    Block<BITS> blk;
    uint32_t scale;
    load_block<BITS>(packed + (size_t)tile * Format<BITS>::kTileBytes, lane, blk, scale);
    float kk[kBlockValues];
    decode_block<BITS>(blk, kk);
    const float dd = scale_f32(scale) * (1.0f / (1 << Format<BITS>::kShift));
    float v[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) v[i] = kk[i] * dd;
    store_tile_values<DT>(lds[wave], lane, v, y + (size_t)tile * (kTileValues * 2));
  }
}

// ---------------------------------------------------------------------------
// fused compressed-domain reduction
// ---------------------------------------------------------------------------

struct ReduceArgs {
  const uint8_t* ranks[QR_MAX_RANKS];
  uint8_t* out;
  uint8_t* y;
  int R;
  int ntiles;
};

template <int BITS, int DT, int RMAX, bool WITH_Y>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
  __shared__ u32x4 lds[WITH_Y ? kWavesPerGroup : 1][WITH_Y ? kChunks : 1];
  constexpr int TB = Format<BITS>::kTileBytes;
  constexpr float kInvShift = 1.0f / (1 << Format<BITS>::kShift);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < a.ntiles; tile += gridDim.x * kWavesPerGroup) {
    const size_t toff = (size_t)tile * TB;
    Block<BITS> blk[RMAX];
    uint32_t sc[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r)
      if (r < a.R) load_block<BITS>(a.ranks[r] + toff, lane, blk[r], sc[r]);
    // exact decode of every rank, fp32 sum in rank order
    float s[kBlockValues];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < a.R) {
        float kk[kBlockValues];
        decode_block<BITS>(blk[r], kk);
        const float dd = scale_f32(sc[r]) * kInvShift;
        if (r == 0) {
#pragma unroll
          for (int i = 0; i < kBlockValues; ++i) s[i] = kk[i] * dd;
        } else {
#pragma unroll
          for (int i = 0; i < kBlockValues; ++i) s[i] = __builtin_fmaf(kk[i], dd, s[i]);
        }
      }
    }
    // round the sum to the I/O dtype, re-encode
    float z[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) z[i] = round_to_dtype<DT>(s[i]);
    Block<BITS> ob;
    float k[kBlockValues];
    const uint32_t scale = encode_block<BITS>(z, ob, k);
    store_block<BITS>(a.out + toff, lane, ob, scale);
    if constexpr (WITH_Y) {
      const float d = scale_f32(scale);
      float v[kBlockValues];
#pragma unroll
      for (int i = 0; i < kBlockValues; ++i) v[i] = k[i] * d;
      store_tile_values<DT>(lds[wave], lane, v, a.y + (size_t)tile * (kTileValues * 2));
    }
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------

inline dim3 grid_for(size_t ntiles) {
  size_t g = (ntiles + kWavesPerGroup - 1) / kWavesPerGroup;
  if (g > (size_t)kMaxGroups) g = kMaxGroups;
  if (g < 1) g = 1;
  return dim3((unsigned)g);
}

template <int BITS>
qr_status launch_encode(int dt, const void* x, void* p, size_t ntiles, hipStream_t st) {
  const dim3 grid = grid_for(ntiles);
  if (dt == kFp16)
    hipLaunchKernelGGL((encode_kernel<BITS, kFp16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)p, (int)ntiles);
  else
    hipLaunchKernelGGL((encode_kernel<BITS, kBf16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)p, (int)ntiles);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_ERR_HIP;
}

template <int BITS>
qr_status launch_decode(int dt, const void* p, void* y, size_t ntiles, hipStream_t st) {
  const dim3 grid = grid_for(ntiles);
  if (dt == kFp16)
    hipLaunchKernelGGL((decode_kernel<BITS, kFp16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)p, (uint8_t*)y, (int)ntiles);
  else
    hipLaunchKernelGGL((decode_kernel<BITS, kBf16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)p, (uint8_t*)y, (int)ntiles);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_ERR_HIP;
}

template <int BITS, int DT, int RMAX>
void launch_reduce_r(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  if (a.y)
    hipLaunchKernelGGL((reduce_kernel<BITS, DT, RMAX, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((reduce_kernel<BITS, DT, RMAX, false>), grid, dim3(kThreads), 0, st, a);
}

template <int BITS, int DT>
void launch_reduce_dt(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  if (a.R <= 1) launch_reduce_r<BITS, DT, 1>(a, grid, st);
  else if (a.R <= 2) launch_reduce_r<BITS, DT, 2>(a, grid, st);
  else if (a.R <= 4) launch_reduce_r<BITS, DT, 4>(a, grid, st);
  else if (a.R <= 8) launch_reduce_r<BITS, DT, 8>(a, grid, st);
  else launch_reduce_r<BITS, DT, 16>(a, grid, st);
}

template <int BITS>
qr_status launch_reduce(int dt, const ReduceArgs& a, hipStream_t st) {
  const dim3 grid = grid_for((size_t)a.ntiles);
  if (dt == kFp16) launch_reduce_dt<BITS, kFp16>(a, grid, st);
  else launch_reduce_dt<BITS, kBf16>(a, grid, st);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_ERR_HIP;
}

// ---------------------------------------------------------------------------
// host-side argument checks (no HIP call)
// ---------------------------------------------------------------------------

inline int tile_bytes(int fmt) {
  switch (fmt) {
    case QR_INT3: return Format<3>::kTileBytes;
    case QR_INT4: return Format<4>::kTileBytes;
    case QR_INT8: return Format<8>::kTileBytes;
    default: return 0;
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Too many tiles for the kernels' int tile index.
inline bool too_large(size_t n) { return n / kTileValues > (size_t)0x7fffffff; }

}  // namespace qr

using namespace qr;

extern "C" {

size_t qr_packed_bytes(qr_format fmt, size_t n) {
  const int tb = tile_bytes(fmt);
  if (!tb || n % kTileValues) return 0;
  return n / kTileValues * (size_t)tb;
}

qr_status qr_encode(qr_format fmt, qr_dtype dtype, const void* x, void* packed, size_t n, void* stream) {
  if (!tile_bytes(fmt) || (dtype != QR_FP16 && dtype != QR_BF16)) return QR_ERR_UNSUPPORTED;
  if (n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (n == 0) return QR_OK;
  if (!x || !packed) return QR_ERR_ARG;
  if (!aligned16(x) || !aligned16(packed)) return QR_ERR_ALIGN;
  const size_t pb = qr_packed_bytes(fmt, n);
  if (overlap(x, 2 * n, packed, pb)) return QR_ERR_ALIAS;
  const size_t nt = n / kTileValues;
  hipStream_t st = (hipStream_t)stream;
  switch (fmt) {
    case QR_INT3: return launch_encode<3>(dtype, x, packed, nt, st);
    case QR_INT4: return launch_encode<4>(dtype, x, packed, nt, st);
    default: return launch_encode<8>(dtype, x, packed, nt, st);
  }
}

qr_status qr_decode(qr_format fmt, qr_dtype dtype, const void* packed, void* y, size_t n, void* stream) {
  if (!tile_bytes(fmt) || (dtype != QR_FP16 && dtype != QR_BF16)) return QR_ERR_UNSUPPORTED;
  if (n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (n == 0) return QR_OK;
  if (!packed || !y) return QR_ERR_ARG;
  if (!aligned16(packed) || !aligned16(y)) return QR_ERR_ALIGN;
  const size_t pb = qr_packed_bytes(fmt, n);
  if (overlap(y, 2 * n, packed, pb)) return QR_ERR_ALIAS;
  const size_t nt = n / kTileValues;
  hipStream_t st = (hipStream_t)stream;
  switch (fmt) {
    case QR_INT3: return launch_decode<3>(dtype, packed, y, nt, st);
    case QR_INT4: return launch_decode<4>(dtype, packed, y, nt, st);
    default: return launch_decode<8>(dtype, packed, y, nt, st);
  }
}

qr_status qr_reduce_compressed(qr_format fmt, qr_dtype dtype, const void* const* packed_ranks, int R,
                               void* packed_out, void* y_out, size_t n, void* stream) {
  if (!tile_bytes(fmt) || (dtype != QR_FP16 && dtype != QR_BF16)) return QR_ERR_UNSUPPORTED;
  if (R < 1 || R > QR_MAX_RANKS) return QR_ERR_ARG;
  if (n % kTileValues || too_large(n)) return QR_ERR_SIZE;
  if (n == 0) return QR_OK;
  if (!packed_ranks || !packed_out) return QR_ERR_ARG;
  for (int r = 0; r < R; ++r)
    if (!packed_ranks[r]) return QR_ERR_ARG;
  for (int r = 0; r < R; ++r)
    if (!aligned16(packed_ranks[r])) return QR_ERR_ALIGN;
  if (!aligned16(packed_out) || (y_out && !aligned16(y_out))) return QR_ERR_ALIGN;
  const size_t pb = qr_packed_bytes(fmt, n);
  for (int r = 0; r < R; ++r) {
    if (overlap(packed_ranks[r], pb, packed_out, pb)) return QR_ERR_ALIAS;
    if (y_out && overlap(packed_ranks[r], pb, y_out, 2 * n)) return QR_ERR_ALIAS;
  }
  if (y_out && overlap(packed_out, pb, y_out, 2 * n)) return QR_ERR_ALIAS;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int r = 0; r < R; ++r) a.ranks[r] = (const uint8_t*)packed_ranks[r];
  a.out = (uint8_t*)packed_out;
  a.y = (uint8_t*)y_out;
  a.R = R;
  a.ntiles = (int)(n / kTileValues);
  hipStream_t st = (hipStream_t)stream;
  switch (fmt) {
    case QR_INT3: return launch_reduce<3>(dtype, a, st);
    case QR_INT4: return launch_reduce<4>(dtype, a, st);
    default: return launch_reduce<8>(dtype, a, st);
  }
}

const char* qr_status_string(qr_status s) {
  switch (s) {
    case QR_OK: return "ok";
    case QR_ERR_ARG: return "invalid argument (null pointer or rank count)";
    case QR_ERR_SIZE: return "value count is not a multiple of 2048";
    case QR_ERR_ALIGN: return "buffer pointer is not 16-byte aligned";
    case QR_ERR_UNSUPPORTED: return "unsupported format or dtype";
    case QR_ERR_ALIAS: return "output buffer overlaps another buffer";
    case QR_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

}  // extern "C"
