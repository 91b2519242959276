// qr_kernels.hpp -- gfx950 kernels and their launch helpers (the C ABI that
// calls them is in qr_api.hip; mixed-format reduce instantiations are in
// qr_reduce_mixed.hip).
//
// Three kernels, each with one 64-lane wave per 2048-value tile and one lane
// per 32-value block (the codec itself is in qr_codec.hpp):
//   encode  fp16/bf16 tile -> LDS (row order) -> lane block -> packed tile
//   decode  packed block -> lane -> LDS (block order) -> fp16/bf16 tile
//   reduce  R packed blocks -> exact fp32 decode + rank-order sum -> round to
//           dtype -> re-encode (packed_out) -> decode (y_out, through LDS);
//           the inputs and the re-encoded sum may use different formats
// The reduce is the in-segment reduction + re-quantization of the two-shot
// all-reduce ("QuickReduce INT3 quantization and benchmarking on MI355",
// "Quantization and Dequantization Paths"; "Flash Communication" review,
// key_machinery): two quantization round trips, decode-sum-encode fused so
// that the fp32 sum never leaves registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qr.h"
#include "qr_codec.hpp"

namespace qr {

// Launch shape: waves (tiles in flight) per workgroup and the grid cap above
// which waves loop over further tiles (grid-stride).
#ifndef QR_WAVES_PER_GROUP
#define QR_WAVES_PER_GROUP 4
#endif
#ifndef QR_MAX_GROUPS
#define QR_MAX_GROUPS (1 << 20)
#endif
// Non-temporal hints per kernel and direction (1 = streamed, 0 = cached).
#ifndef QR_ENC_NT_LOAD
#define QR_ENC_NT_LOAD 1
#endif
#ifndef QR_ENC_NT_STORE
#define QR_ENC_NT_STORE 1
#endif
#ifndef QR_DEC_NT_LOAD
#define QR_DEC_NT_LOAD 0
#endif
#ifndef QR_DEC_NT_STORE
#define QR_DEC_NT_STORE 1
#endif
#ifndef QR_RED_NT_LOAD
#define QR_RED_NT_LOAD 1
#endif
#ifndef QR_RED_NT_STORE
#define QR_RED_NT_STORE 1
#endif
// Tiles each encode wave processes (the next one prefetched while encoding).
#ifndef QR_ENC_TILES_PER_WAVE
#define QR_ENC_TILES_PER_WAVE 1
#endif
// Encode mapping: 0 = lane per 32-value block through an LDS transpose,
// 1 = lane per 8-value unit with a 4-lane DPP block maximum.
#ifndef QR_ENC_QUAD
#define QR_ENC_QUAD 0
#endif
// 1: issue every rank's loads before decoding; 0: let the scheduler pipeline them.
#ifndef QR_RED_LOADS_FIRST
#define QR_RED_LOADS_FIRST 1
#endif
constexpr int kWavesPerGroup = QR_WAVES_PER_GROUP;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kMaxGroups = QR_MAX_GROUPS;

// ---------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void encode_kernel(const uint8_t* __restrict__ x,
                                                          uint8_t* __restrict__ packed, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kChunks];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  u32x4* tl = lds[wave];
  const int stride = gridDim.x * kWavesPerGroup;
  int tile = blockIdx.x * kWavesPerGroup + wave;
  if (tile >= ntiles) return;
  // the next tile's 4 KB is loaded into registers while this one is encoded
  u32x4 v[4];
  auto load_tile = [&](int t) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)t * (kTileValues * 2));
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ld<QR_ENC_NT_LOAD>(src + lane + kWave * k);
  };
  load_tile(tile);
  for (; tile < ntiles; tile += stride) {
#pragma unroll
    for (int k = 0; k < 4; ++k) tl[swz(lane + kWave * k)] = v[k];
    if (tile + stride < ntiles) load_tile(tile + stride);
    wave_lds_sync();
    uint32_t w[kBlockValues / 2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 c = tl[swz(4 * lane + j)];
      w[4 * j] = c.x; w[4 * j + 1] = c.y; w[4 * j + 2] = c.z; w[4 * j + 3] = c.w;
    }
    wave_lds_sync();  // the next tile overwrites this LDS tile
    uint32_t t[kBlockValues];
    const uint32_t scale = quantize_words<BITS, DT>(w, t);
    Block<BITS> blk;
    pack_block<BITS>(t, blk);
    store_block<BITS, QR_ENC_NT_STORE>(packed + (size_t)tile * Format<BITS>::kTileBytes, lane, blk, scale);
  }
}

// Alternative encode mapping: lane = one 8-value unit (a coalesced 16-byte
// load straight into registers), four lanes per block; the block maximum is
// reduced across the 4-lane group with DPP quad permutes and every lane of
// the group derives the same scale.  No LDS.
__device__ __forceinline__ float quad_max(float m) {
  // quad_perm [1,0,3,2] then [2,3,0,1]
  m = __builtin_fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0xB1, 0xF, 0xF, false)));
  m = __builtin_fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0x4E, 0xF, 0xF, false)));
  return m;
}

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void encode_quad_kernel(const uint8_t* __restrict__ x,
                                                               uint8_t* __restrict__ packed, int ntiles) {
  constexpr int TB = Format<BITS>::kTileBytes;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < ntiles; tile += gridDim.x * kWavesPerGroup) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + (size_t)tile * (kTileValues * 2));
    uint8_t* dst = packed + (size_t)tile * TB;
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ld<QR_ENC_NT_LOAD>(src + lane + kWave * k);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = kWave * k + lane;  // unit index in the tile
      const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
      float z[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        z[2 * q] = lo_to_f32<DT>(w[q]);
        z[2 * q + 1] = hi_to_f32<DT>(w[q]);
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(z[i]));
      m = quad_max(m);
      float d, e;
      const uint32_t scale = block_scale<BITS>(m, d, e);
      uint32_t t[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] = quantize<BITS>(z[i] * e);
      if constexpr (BITS == 4) {
        st<QR_ENC_NT_STORE>(pack_int4_unit(t), reinterpret_cast<uint32_t*>(dst + 4 * u));
      } else if constexpr (BITS == 8) {
        st<QR_ENC_NT_STORE>(u32x2{pack_int8_word(t), pack_int8_word(t + 4)}, reinterpret_cast<u32x2*>(dst + 8 * u));
      } else {
        // bytes c0 c2 c4 c6 and c1 c3 c5 c7 -> 2-bit plane word and 1-bit plane byte
        const uint32_t ev = lo_pair(t[0], t[2]) | hi_pair(t[4], t[6]);
        const uint32_t od = lo_pair(t[1], t[3]) | hi_pair(t[5], t[7]);
        const uint32_t nib = ev | (od << 4);           // nibble j = code j (INT4 order)
        uint32_t lo = nib & 0x33333333u;               // low pairs at bits 4j
        lo = (lo | (lo >> 2)) & 0x0F0F0F0Fu;
        lo = (lo | (lo >> 4)) & 0x00FF00FFu;
        lo = (lo | (lo >> 8)) & 0x0000FFFFu;
        uint32_t hb = (nib >> 2) & 0x11111111u;        // high bits at bits 4j
        hb = (hb | (hb >> 3)) & 0x03030303u;
        hb = (hb | (hb >> 6)) & 0x000F000Fu;
        hb = (hb | (hb >> 12)) & 0x000000FFu;
        st<QR_ENC_NT_STORE>((uint16_t)lo, reinterpret_cast<uint16_t*>(dst + 2 * u));
        st<QR_ENC_NT_STORE>((uint8_t)hb, dst + Format<3>::kHighOffset + u);
      }
      if ((lane & 3) == 0)
        st<QR_ENC_NT_STORE>((uint16_t)scale, reinterpret_cast<uint16_t*>(dst + Format<BITS>::kScaleOffset + 2 * (u >> 2)));
    }
  }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// One lane's 32 output values (block order) into the wave's LDS tile.
template <int DT>
__device__ __forceinline__ void write_lane_values(u32x4* tl, int lane, const float (&y)[kBlockValues]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    u32x4 c;
    c.x = pack2<DT>(y[8 * j + 0], y[8 * j + 1]);
    c.y = pack2<DT>(y[8 * j + 2], y[8 * j + 3]);
    c.z = pack2<DT>(y[8 * j + 4], y[8 * j + 5]);
    c.w = pack2<DT>(y[8 * j + 6], y[8 * j + 7]);
    tl[swz(4 * lane + j)] = c;
  }
}

// The wave's LDS tile to global memory in row order (coalesced 16-byte stores).
template <bool NT>
__device__ __forceinline__ void flush_tile(u32x4* tl, int lane, uint8_t* __restrict__ dst) {
  wave_lds_sync();
  u32x4* out = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int k = 0; k < 4; ++k) st<NT>(tl[swz(lane + kWave * k)], out + lane + kWave * k);
  wave_lds_sync();
}

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ y, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kChunks];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < ntiles; tile += gridDim.x * kWavesPerGroup) {
    Block<BITS> blk;
    uint32_t scale;
    load_block<BITS, QR_DEC_NT_LOAD>(packed + (size_t)tile * Format<BITS>::kTileBytes, lane, blk, scale);
    float kk[kBlockValues];
    decode_block<BITS>(blk, kk);
    const float dd = scale_f32(scale) * (1.0f / (1 << Format<BITS>::kShift));
    float v[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) v[i] = kk[i] * dd;
    write_lane_values<DT>(lds[wave], lane, v);
    flush_tile<QR_DEC_NT_STORE>(lds[wave], lane, y + (size_t)tile * (kTileValues * 2));
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

template <int BI, int BO, int DT, int R, bool WITH_Y>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
  __shared__ u32x4 lds[WITH_Y ? kWavesPerGroup : 1][WITH_Y ? kChunks : 1];
  constexpr int TB = Format<BI>::kTileBytes;    // input tiles
  constexpr int TBO = Format<BO>::kTileBytes;   // re-encoded tiles
  constexpr float kInvShift = 1.0f / (1 << Format<BI>::kShift);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < a.ntiles; tile += gridDim.x * kWavesPerGroup) {
    const size_t toff = (size_t)tile * TB;
    Block<BI> blk[R];
    uint32_t sc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) load_block<BI, QR_RED_NT_LOAD>(a.ranks[r] + toff, lane, blk[r], sc[r]);
#if QR_RED_LOADS_FIRST
    __builtin_amdgcn_sched_barrier(0);  // every rank's loads in flight before decoding starts
#endif
    // exact decode of every rank, fp32 sum in rank order: s = y_0, s = s + y_r
    float s[kBlockValues];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float kk[kBlockValues];
      decode_block<BI>(blk[r], kk);
      const float dd = scale_f32(sc[r]) * kInvShift;
      if (r == 0) {
#pragma unroll
        for (int i = 0; i < kBlockValues; ++i) s[i] = kk[i] * dd;
      } else {
#pragma unroll
        for (int i = 0; i < kBlockValues; ++i) s[i] = __builtin_fmaf(kk[i], dd, s[i]);
      }
    }
    // re-encode dtype_RNE(s): rounding is monotonic and symmetric, so the
    // block maximum of the rounded values is the rounded maximum of |s|
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(s[i]));
    float d, e;
    const uint32_t scale = block_scale<BO>(round_to_dtype<DT>(m), d, e);
    uint32_t t[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; i += 2) {
      float v0, v1;
      round_scale2<DT>(s[i], s[i + 1], e, v0, v1);
      t[i] = quantize<BO>(v0);
      t[i + 1] = quantize<BO>(v1);
    }
    if constexpr (WITH_Y) {  // decode of the re-encoded sum, straight from the codes
      float v[kBlockValues];
#pragma unroll
      for (int i = 0; i < kBlockValues; ++i) v[i] = code_value<BO>(t[i]) * d;
      write_lane_values<DT>(lds[wave], lane, v);
    }
    Block<BO> ob;
    pack_block<BO>(t, ob);
    store_block<BO, QR_RED_NT_STORE>(a.out + (size_t)tile * TBO, lane, ob, scale);
    if constexpr (WITH_Y) flush_tile<QR_RED_NT_STORE>(lds[wave], lane, a.y + (size_t)tile * (kTileValues * 2));
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
  const dim3 grid = grid_for((ntiles + QR_ENC_TILES_PER_WAVE - 1) / QR_ENC_TILES_PER_WAVE);
#if QR_ENC_QUAD
#define QR_ENCODE_KERNEL encode_quad_kernel
#else
#define QR_ENCODE_KERNEL encode_kernel
#endif
  if (dt == kFp16)
    hipLaunchKernelGGL((QR_ENCODE_KERNEL<BITS, kFp16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)p, (int)ntiles);
  else
    hipLaunchKernelGGL((QR_ENCODE_KERNEL<BITS, kBf16>), grid, dim3(kThreads), 0, st,
                       (const uint8_t*)x, (uint8_t*)p, (int)ntiles);
#undef QR_ENCODE_KERNEL
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

template <int BI, int BO, int DT, int R>
void launch_reduce_r(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  if (a.y)
    hipLaunchKernelGGL((reduce_kernel<BI, BO, DT, R, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((reduce_kernel<BI, BO, DT, R, false>), grid, dim3(kThreads), 0, st, a);
}

template <int BI, int BO, int DT>
void launch_reduce_dt(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  switch (a.R) {
#define QR_RANK_CASE(r) \
  case r: launch_reduce_r<BI, BO, DT, r>(a, grid, st); break;
    QR_RANK_CASE(1) QR_RANK_CASE(2) QR_RANK_CASE(3) QR_RANK_CASE(4)
    QR_RANK_CASE(5) QR_RANK_CASE(6) QR_RANK_CASE(7) QR_RANK_CASE(8)
    QR_RANK_CASE(9) QR_RANK_CASE(10) QR_RANK_CASE(11) QR_RANK_CASE(12)
    QR_RANK_CASE(13) QR_RANK_CASE(14) QR_RANK_CASE(15) QR_RANK_CASE(16)
#undef QR_RANK_CASE
    default: break;  // R was validated to be in [1, QR_MAX_RANKS]
  }
}

template <int BI, int BO>
qr_status launch_reduce(int dt, const ReduceArgs& a, hipStream_t st) {
  const dim3 grid = grid_for((size_t)a.ntiles);
  if (dt == kFp16) launch_reduce_dt<BI, BO, kFp16>(a, grid, st);
  else launch_reduce_dt<BI, BO, kBf16>(a, grid, st);
  return hipGetLastError() == hipSuccess ? QR_OK : QR_ERR_HIP;
}

// Reduce with input format != output format (instantiated in qr_reduce_mixed.hip,
// one object per input format).
qr_status launch_reduce_mixed_from3(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
qr_status launch_reduce_mixed_from4(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
qr_status launch_reduce_mixed_from8(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);

}  // namespace qr
