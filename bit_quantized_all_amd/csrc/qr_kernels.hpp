// qr_kernels.hpp -- gfx950 kernels and their launch helpers (the C ABI that
// calls them is in qr_api.hip; the instantiations are spread over
// qr_api.hip (INT3/INT4/INT8), qr_reduce_mixed.hip (mixed INT formats),
// qr_asym.hip (asymmetric formats) and qr_fp4.hip (FP4), so they build in
// parallel).
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
// Cache-policy operands (cache_policy()) of the memory instructions, per
// kernel and direction; the reduce's y output has its own.
#define QR_POL(nt) ((nt) ? kNT : 0)
#ifndef QR_ENC_LOAD_POL
#define QR_ENC_LOAD_POL QR_POL(QR_ENC_NT_LOAD)
#endif
#ifndef QR_ENC_STORE_POL
#define QR_ENC_STORE_POL QR_POL(QR_ENC_NT_STORE)
#endif
#ifndef QR_DEC_LOAD_POL
#define QR_DEC_LOAD_POL QR_POL(QR_DEC_NT_LOAD)
#endif
#ifndef QR_DEC_STORE_POL
#define QR_DEC_STORE_POL QR_POL(QR_DEC_NT_STORE)
#endif
#ifndef QR_RED_LOAD_POL
#define QR_RED_LOAD_POL QR_POL(QR_RED_NT_LOAD)
#endif
#ifndef QR_RED_STORE_POL
#define QR_RED_STORE_POL QR_POL(QR_RED_NT_STORE)
#endif
#ifndef QR_RED_Y_STORE_POL
#define QR_RED_Y_STORE_POL QR_RED_STORE_POL
#endif
// Tiles each encode wave processes (the next one prefetched while encoding).
#ifndef QR_ENC_TILES_PER_WAVE
#define QR_ENC_TILES_PER_WAVE 1
#endif
// 1: issue every rank's loads before decoding; 0: let the scheduler pipeline them.
#ifndef QR_RED_LOADS_FIRST
#define QR_RED_LOADS_FIRST 1
#endif
// registers per lane that the R blocks of codes and scales may hold before
// the decode starts; above it the loads are left to the scheduler
#ifndef QR_RED_LOADS_FIRST_REGS
#define QR_RED_LOADS_FIRST_REGS 128
#endif
// 1: the fused decode of the re-encoded sum builds fp16 outputs as packed
// fp16 pairs (byte permute, packed subtract, packed multiply).
#ifndef QR_Y_HALF_PAIRS
#define QR_Y_HALF_PAIRS 1
#endif
// 1: reduce waves loop over tiles with the next tile's loads in flight
// (grid of QR_RED_GROUPS_PER_CU workgroups per CU); 0: one tile per wave.
// Measured slower and kept off: INT3 R = 2, 134M fp16 values per rank,
// 74.8 -> 88.2 us (4 workgroups per CU) and 87.2 us (6); INT4 R = 8
// 150.9 -> 172.6 us; the second register set also halves the occupancy.
#ifndef QR_RED_PREFETCH
#define QR_RED_PREFETCH 0
#endif
#ifndef QR_RED_GROUPS_PER_CU
#define QR_RED_GROUPS_PER_CU 4
#endif
// Rank-ordered decode: each rank's codes pass an empty asm that depends on
// the previous rank's last running sum, so rank r's decode waits only for the
// loads of ranks 0..r (without it the scheduler hoists every rank's code
// unpacking above the first sum and each wave waits for all its loads at
// once).  It pays when a launch has few waves per SIMD to hide that wait and
// costs a little when it has many.  Measured, reduce per launch, 8 ranks:
//   INT4 (fp16)   8192 tiles 23.6 -> 22.8 us ordered, 16384 41.4 -> 41.0,
//                 32768 78.2 -> 78.3, 65536 (134M values) 150.8 -> 152.0
//   INT4 -> INT8  8192 tiles 24.8 -> 24.4;   INT8 (R = 4) 8192 22.99 -> 22.72
//   FP4           8192 tiles 21.9 -> 22.1;   ASYM4 even
//   INT3 R = 2    65536 tiles 72.4 -> 72.0 (INT3 unpacks two bit planes)
// QR_RED_RANK_ORDER: 0 never, 2 always, 1 (default) INT3 inputs always and
// INT4 / INT8 inputs up to QR_RED_ORDER_MAX_TILES tiles.
#ifndef QR_RED_RANK_ORDER
#define QR_RED_RANK_ORDER 1
#endif
#ifndef QR_RED_ORDER_MAX_TILES
#define QR_RED_ORDER_MAX_TILES 16384
#endif
// 0: the reduce of input format BI is never ordered, 1: always, 2: by size.
template <int BI>
constexpr int kOrderMode =
    QR_RED_RANK_ORDER == 0   ? 0
    : QR_RED_RANK_ORDER == 2 ? 1
    : Format<BI>::kCodeBits == 3 ? 1
    : (!Format<BI>::kAsym && !Format<BI>::kFp4) ? 2
                                                : 0;
// Encode workgroups resident on one CU at a time.  Every encode wave has its
// whole 4 KB input tile in flight at once; a full CU (8 workgroups, 32 waves)
// keeps more requests outstanding than HBM serves best, and 5 workgroups
// (20 waves) measured fastest: per 134M-value fp16 rank, INT4 56.9 -> 53.2 us,
// INT3 53.9 -> 51.1 us, INT8 64.4 -> 62.6 us; 3 and 2 workgroups were slower.
// The launch adds dynamic LDS so that no more fit in the CU's 160 KB
// (residency_pad(); caps of 3 and more, which keep a workgroup's LDS within
// 64 KB).
#ifndef QR_ENC_GROUPS_PER_CU
#define QR_ENC_GROUPS_PER_CU 5
#endif
// Reduce workgroups resident on one CU at a time (0: as many as registers
// allow), set the same way.  The fused reduce writes more than it reads
// (y alone is 2 bytes per value); with fewer waves in flight HBM serves its
// mix of reads and writes better: INT3 R = 2, 134M fp16 values per rank,
// 74.9 -> 72.2 us at 5 workgroups (20 waves), 72.6 us at 6; INT3 R = 4 at
// 512 MiB per rank 189.5 -> 182.3 us.  Kernels whose registers already allow
// at most 20 waves per CU (INT4 R = 8 unordered: 143 VGPRs, 12 waves) are
// not limited further.
#ifndef QR_RED_GROUPS_PER_CU_MAX
#define QR_RED_GROUPS_PER_CU_MAX 5
#endif
// The same for reduces of 8-bit inputs, whose waves each have twice the
// input bytes in flight: INT8 R = 4, 268M fp16 values per rank, 315.7 ->
// 310.3 us at 3 workgroups (4: 315.3); 67M values 79.7 -> 79.3 us.
#ifndef QR_RED8_GROUPS_PER_CU_MAX
#define QR_RED8_GROUPS_PER_CU_MAX 3
#endif
// Decode workgroups resident on one CU at a time (0: no limit); per
// 134M-value INT4 fp16 rank 56.4 -> 53.8 us at 5 workgroups (20 waves).
#ifndef QR_DEC_GROUPS_PER_CU_MAX
#define QR_DEC_GROUPS_PER_CU_MAX 5
#endif
static_assert(QR_ENC_GROUPS_PER_CU == 0 || QR_ENC_GROUPS_PER_CU >= 3, "residency caps of 3 or more");
static_assert(QR_RED_GROUPS_PER_CU_MAX == 0 || QR_RED_GROUPS_PER_CU_MAX >= 3, "residency caps of 3 or more");
static_assert(QR_RED8_GROUPS_PER_CU_MAX == 0 || QR_RED8_GROUPS_PER_CU_MAX >= 3, "residency caps of 3 or more");
static_assert(QR_DEC_GROUPS_PER_CU_MAX == 0 || QR_DEC_GROUPS_PER_CU_MAX >= 3, "residency caps of 3 or more");
constexpr int kWavesPerGroup = QR_WAVES_PER_GROUP;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kMaxGroups = QR_MAX_GROUPS;
constexpr int kLdsBytesPerCU = 160 * 1024;

// The caps above apply to launches of more than QR_CAP_MIN_GROUPS workgroups
// per CU.  A smaller grid runs in at most two generations of full residency,
// and there a cap only adds generations: 8192 tiles (8 workgroups per CU)
// encode in 8.5 us uncapped against 9.1 us at 5, and decode in 7.4 against
// 9.3 us (INT4 fp16); at 16384 tiles uncapped is 0.6% (encode) and 1.3%
// (decode) faster.
#ifndef QR_CAP_MIN_GROUPS
#define QR_CAP_MIN_GROUPS 16
#endif

// 16-byte LDS chunks per wave that the encode and decode kernels use (the
// wave's tile); a residency cap adds dynamic LDS at launch (residency_pad()).
constexpr int kEncLdsChunks = kTileSlots;
constexpr int kDecLdsChunks = kTileSlots;

// 1: workgroups of formats whose tiles are not whole 128-byte cache lines
// take their tiles in XCD pairs (group_index()); 0: in dispatch order.
#ifndef QR_XCD_PAIRS
#define QR_XCD_PAIRS 1
#endif
// The same for the encode (1), or dispatch order there (0): the pairing made
// the ASYM4 encode 1.1% slower (53.29 -> 52.71 us per 134M fp16 values
// without it); the reduce keeps it (154.8 -> 154.2 us with it).
#ifndef QR_ENC_XCD_PAIRS
#define QR_ENC_XCD_PAIRS 0
#endif

// Index, in tile order, of workgroup b of a grid of `grid`.  Workgroups are
// dealt to the 8 XCDs in turn (workgroup b runs on XCD b % 8), each with its
// own L2.  When a tile is not a whole number of 128-byte lines (TB1 or TB2
// bytes), adjacent tiles share a line, and only the boundaries of aligned
// groups of 8 tiles fall on line boundaries.  The two workgroups (of 4 tiles
// each) that cover such a group are then workgroups b and b + 8 of a window of
// 16, which run on one XCD, so that no line is split between two L2s.  The
// last, partial window keeps the dispatch order.
template <int TB1, int TB2, bool PAIRS = QR_XCD_PAIRS>
__device__ __forceinline__ int group_index(int b, int grid) {
  if constexpr (!PAIRS || kWavesPerGroup != 4 || (TB1 % 128 == 0 && TB2 % 128 == 0)) {
    return b;
  } else {
    static_assert((8 * TB1) % 128 == 0 && (8 * TB2) % 128 == 0, "8 tiles span whole lines");
    const int win = b & ~15;
    if (win + 16 > grid) return b;
    const int r = b & 15;
    return win + 2 * (r & 7) + (r >> 3);
  }
}

// ---------------------------------------------------------------------------
// encode
// ---------------------------------------------------------------------------

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void encode_kernel(const uint8_t* __restrict__ x,
                                                          uint8_t* __restrict__ packed, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kEncLdsChunks];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  u32x4* tl = lds[wave];
  const int stride = gridDim.x * kWavesPerGroup;
  constexpr int TB = Format<BITS>::kTileBytes;
  int tile = group_index<TB, TB, QR_XCD_PAIRS && QR_ENC_XCD_PAIRS>(blockIdx.x, gridDim.x) * kWavesPerGroup + wave;
  if (tile >= ntiles) return;
  // the next tile's 4 KB is loaded into registers while this one is encoded
  u32x4 v[4];
  auto load_tile = [&](int t) {
    const TileRef src = tile_ref(x + (size_t)t * (kTileValues * 2), kTileValues * 2);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = ld16<QR_ENC_LOAD_POL>(src, 16 * (lane + kWave * k));
  };
  load_tile(tile);
  for (; tile < ntiles; tile += stride) {
#pragma unroll
    for (int k = 0; k < 4; ++k) tl[row_slot(lane, k)] = v[k];
    if (tile + stride < ntiles) load_tile(tile + stride);
    wave_lds_sync();
    uint32_t w[kBlockValues / 2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 c = tl[block_slot(lane, j)];
      w[4 * j] = c.x; w[4 * j + 1] = c.y; w[4 * j + 2] = c.z; w[4 * j + 3] = c.w;
    }
    wave_lds_sync();  // the next tile overwrites this LDS tile
    uint32_t scale;
    Block<BITS> blk;
    if constexpr (Format<BITS>::kFp4) {
      scale = quantize_words_fp4<DT>(w, blk);
    } else {
      uint32_t t[kBlockValues];
      if constexpr (Format<BITS>::kAsym)
        scale = quantize_words_asym<BITS, DT>(w, t);
      else
        scale = quantize_words<BITS, DT>(w, t);
      pack_block<BITS>(t, blk);
    }
    const TileRef tp = tile_ref(packed + (size_t)tile * Format<BITS>::kTileBytes, Format<BITS>::kTileBytes);
    if constexpr (kStaged<BITS>) stage_codes_out<QR_ENC_STORE_POL>(tl, lane, blk, tp);
    store_block<BITS, QR_ENC_STORE_POL>(tp, lane, blk, scale);
  }
}

// 1: INT3 and INT4 encode with an 8-lane group per 32-value block (4 values
// per lane): the block maximum is a three-step DPP reduction over the group,
// every lane derives the scale, and the packed tile is assembled in LDS from
// each lane's bits, then stored coalesced.  0: one lane per block (the
// default).  Measured slower; kept for comparison.
#ifndef QR_ENC_GROUP8
#define QR_ENC_GROUP8 0
#endif

// Maximum of v over the 8 lanes of an aligned group (DPP quad permutes
// [1,0,3,2], [2,3,0,1], then the half-row mirror lane i <-> 7 - i).
__device__ __forceinline__ int group8_max_i32(int v) {
  v = __builtin_elementwise_max(v, __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
  v = __builtin_elementwise_max(v, __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));
  return __builtin_elementwise_max(v, __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false));
}

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void encode_group8_kernel(const uint8_t* __restrict__ x,
                                                                 uint8_t* __restrict__ packed, int ntiles) {
  static_assert(BITS == 3 || BITS == 4, "symmetric 3- and 4-bit codes");
  constexpr int TB = Format<BITS>::kTileBytes;
  __shared__ u32x4 lds[kWavesPerGroup][kEncLdsChunks];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  u32x4* tl = lds[wave];
  uint8_t* sb = reinterpret_cast<uint8_t*>(tl);
  for (int tile = blockIdx.x * kWavesPerGroup + wave; tile < ntiles; tile += gridDim.x * kWavesPerGroup) {
    const TileRef src = tile_ref(x + (size_t)tile * (kTileValues * 2), kTileValues * 2);
    u32x2 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ld8<QR_ENC_LOAD_POL>(src, 512 * i + 8 * lane);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // values 256 i + 4 lane .. + 3: block 8 i + lane / 8, unit 32 i + lane / 2
      const uint32_t w[2] = {v[i].x, v[i].y};
      u16x2 m2 = __builtin_elementwise_max(__builtin_bit_cast(u16x2, w[0] & 0x7fff7fffu),
                                            __builtin_bit_cast(u16x2, w[1] & 0x7fff7fffu));
      const int mb = group8_max_i32(m2.x > m2.y ? m2.x : m2.y);
      float d, e;
      const uint32_t sbits = block_scale<BITS>(half_pattern_to_f32<DT>((uint32_t)mb), d, e);
      uint32_t t[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float v0, v1;
        scale_pair<DT>(w[j], e, v0, v1);
        t[2 * j] = quantize<BITS>(v0);
        t[2 * j + 1] = quantize<BITS>(v1);
      }
      const uint32_t c = lo_pair(t[0], t[1]) | hi_pair(t[2], t[3]);  // bytes q0 q1 q2 q3
      const uint32_t unit = 32 * i + (lane >> 1);
      if constexpr (BITS == 4) {
        const uint32_t h = (c & 0xFu) | ((c >> 4) & 0xF0u) | ((c >> 8) & 0xF00u) | ((c >> 12) & 0xF000u);
        *reinterpret_cast<uint16_t*>(sb + 4 * unit + 2 * (lane & 1)) = (uint16_t)h;
      } else {
        const uint32_t lo = (c & 3u) | ((c >> 6) & 0xCu) | ((c >> 12) & 0x30u) | ((c >> 18) & 0xC0u);
        const uint32_t hi = ((c >> 2) & 1u) | ((c >> 9) & 2u) | ((c >> 16) & 4u) | ((c >> 23) & 8u);
        sb[2 * unit + (lane & 1)] = (uint8_t)lo;
        const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)hi, 0xB1, 0xF, 0xF, false);
        sb[Format<3>::kHighOffset + unit] = (uint8_t)((lane & 1) ? (other | (hi << 4)) : (hi | (other << 4)));
      }
      if ((lane & 7) == 0)
        *reinterpret_cast<uint16_t*>(sb + Format<BITS>::kScaleOffset + 2 * (8 * i + (lane >> 3))) = (uint16_t)sbits;
    }
    wave_lds_sync();
    const TileRef tp = tile_ref(packed + (size_t)tile * TB, TB);
#pragma unroll
    for (int k = 0; k < (TB + 16 * kWave - 1) / (16 * kWave); ++k)
      st16<QR_ENC_STORE_POL>(tp, 16 * (lane + kWave * k), tl[lane + kWave * k]);  // past the tile: dropped
    wave_lds_sync();
  }
}

// ---------------------------------------------------------------------------
// decode
// ---------------------------------------------------------------------------

// One lane's 32 output values (block order, as 16 packed dtype pairs) into
// the wave's LDS tile.
__device__ __forceinline__ void write_lane_words(u32x4* tl, uint32_t lane, const uint32_t (&w)[kBlockValues / 2]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) tl[block_slot(lane, j)] = u32x4{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
}

// The same from 32 fp32 values, each rounded to the dtype (nearest even).
template <int DT>
__device__ __forceinline__ void write_lane_values(u32x4* tl, uint32_t lane, const float (&y)[kBlockValues]) {
  uint32_t w[kBlockValues / 2];
#pragma unroll
  for (int i = 0; i < kBlockValues / 2; ++i) w[i] = pack2<DT>(y[2 * i], y[2 * i + 1]);
  write_lane_words(tl, lane, w);
}

// The wave's LDS tile to global memory in row order (coalesced 16-byte stores).
template <int NT>
__device__ __forceinline__ void flush_tile(u32x4* tl, uint32_t lane, TileRef dst) {
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 4; ++k) st16<NT>(dst, 16 * (lane + kWave * k), tl[row_slot(lane, k)]);
  wave_lds_sync();
}

template <int BITS, int DT>
__global__ __launch_bounds__(kThreads) void decode_kernel(const uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ y, int ntiles) {
  __shared__ u32x4 lds[kWavesPerGroup][kDecLdsChunks];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  constexpr int TB = Format<BITS>::kTileBytes;
  for (int tile = group_index<TB, TB>(blockIdx.x, gridDim.x) * kWavesPerGroup + wave; tile < ntiles;
       tile += gridDim.x * kWavesPerGroup) {
    Block<BITS> blk;
    uint32_t scale;
    load_block<BITS, QR_DEC_LOAD_POL>(tile_ref(packed + (size_t)tile * Format<BITS>::kTileBytes, Format<BITS>::kTileBytes),
                                     lane, blk, scale);
    if constexpr (kStaged<BITS>) stage_codes_in(lds[wave], lane, blk);
    float kk[kBlockValues];
    float dd, ddo;  // scales of even and odd values
    if constexpr (Format<BITS>::kAsym) {
      const AsymMeta am = group_meta<BITS>(scale, lane, meta_sel(lane));
      decode_block_asym<BITS>(blk, am.nz, am.nzo, kk);
      dd = am.d;
      ddo = am.dodd;
    } else if constexpr (Format<BITS>::kFp4) {
      decode_block_fp4(blk, kk);
      dd = ddo = scale_f32(scale);
    } else {
      decode_block<BITS>(blk, kk);
      dd = scale_f32(scale) * (1.0f / (1 << Format<BITS>::kShift));
      ddo = dd;
    }
    float v[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) v[i] = kk[i] * ((i & 1) ? ddo : dd);
    write_lane_values<DT>(lds[wave], lane, v);
    flush_tile<QR_DEC_STORE_POL>(lds[wave], lane, tile_ref(y + (size_t)tile * (kTileValues * 2), kTileValues * 2));
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

// LDS chunks per reduce wave: the fp16/bf16 output tile (WITH_Y) and / or the
// 2 KB staging region of 8-bit codes, which reuses the output tile's space.
template <int BI, int BO, bool WITH_Y>
constexpr int kReduceLdsChunks =
    WITH_Y ? kTileSlots
           : ((kStaged<BI> || kStaged<BO>) ? kStageSlots : ((Format<BI>::kCodeBits == 3 && QR_INT3_LDS_STAGE) ? 64 : 1));

// Every rank's block `lane` of tile `tile` (codes and scale) into registers.
template <int BI, int R>
__device__ __forceinline__ void load_ranks(const ReduceArgs& a, int tile, uint32_t lane, Block<BI> (&blk)[R],
                                           uint32_t (&sc)[R]) {
  const size_t toff = (size_t)tile * Format<BI>::kTileBytes;
#pragma unroll
  for (int r = 0; r < R; ++r)
    load_block<BI, QR_RED_LOAD_POL>(tile_ref(a.ranks[r] + toff, Format<BI>::kTileBytes), lane, blk[r], sc[r]);
}

// Passes a block's registers through an empty asm that also reads `after`:
// code that uses the block is then scheduled after `after` is computed.
template <int CB>
__device__ __forceinline__ void order_after(CodeBlock<CB>& blk, uint32_t& sc, float after) {
  if constexpr (CB == 3) {
    asm volatile("" : "+v"(blk.low[0]), "+v"(blk.low[1]), "+v"(blk.high), "+v"(sc) : "v"(after));
  } else if constexpr (CB == 4) {
    asm volatile("" : "+v"(blk.w[0]), "+v"(blk.w[1]), "+v"(blk.w[2]), "+v"(blk.w[3]), "+v"(sc) : "v"(after));
  } else {
    asm volatile("" : "+v"(blk.w[0]), "+v"(blk.w[1]), "+v"(blk.w[2]), "+v"(blk.w[3]), "+v"(blk.w[4]),
                 "+v"(blk.w[5]), "+v"(blk.w[6]), "+v"(blk.w[7]), "+v"(sc) : "v"(after));
  }
}

// The reduction of one tile whose R blocks are in registers: exact decode,
// fp32 rank-order sum, re-encode into packed_out and (WITH_Y) decode into y.
template <int BI, int BO, int DT, int R, bool WITH_Y, bool ORDER>
__device__ __forceinline__ void reduce_tile(const ReduceArgs& a, int tile, uint32_t lane, u32x4* tl,
                                            Block<BI> (&blk)[R], uint32_t (&sc)[R]) {
  constexpr int TBO = Format<BO>::kTileBytes;   // re-encoded tiles
  constexpr float kInvShift = 1.0f / (1 << Format<BI>::kShift);
  // exact decode of every rank, fp32 sum in rank order: s = y_0, s = s + y_r
  float s[kBlockValues];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    // rank r's codes enter its decode only after rank r - 1 is summed, so the
    // decodes run in load order and each waits only for its own loads
    if constexpr (ORDER)
      if (r > 0) order_after(blk[r], sc[r], s[kBlockValues - 1]);
    if constexpr (kStaged<BI>) stage_codes_in(tl, lane, blk[r]);
    float kk[kBlockValues];
    float dd, ddo;  // scales of even and odd values (exact products with kk)
    if constexpr (Format<BI>::kAsym) {
      const AsymMeta am = group_meta<BI>(sc[r], lane, meta_sel(lane));
      decode_block_asym<BI>(blk[r], am.nz, am.nzo, kk);
      dd = am.d;
      ddo = am.dodd;
    } else if constexpr (Format<BI>::kFp4) {
      decode_block_fp4(blk[r], kk);
      dd = ddo = scale_f32(sc[r]);
    } else {
      decode_block<BI>(blk[r], kk);
      dd = scale_f32(sc[r]) * kInvShift;
      ddo = dd;
    }
    if (r == 0) {
      // fma(k, d, +0) is the exact product k * d up to the sign of a zero
      // (+0 for -0); it lets the fp16 halves of the asymmetric decode feed
      // one mixed-precision FMA.  Asymmetric inputs reduce only into an
      // asymmetric format, whose code of +-0 is z either way, so no later
      // step can observe the difference.
#pragma unroll
      for (int i = 0; i < kBlockValues; ++i) {
        if constexpr (Format<BI>::kAsym)
          s[i] = __builtin_fmaf(kk[i], (i & 1) ? ddo : dd, 0.0f);
        else
          s[i] = kk[i] * dd;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBlockValues; ++i) s[i] = __builtin_fmaf(kk[i], (i & 1) ? ddo : dd, s[i]);
    }
  }
  // re-encode dtype_RNE(s): rounding is monotonic and symmetric, so the
  // block maximum (group range) of the rounded values is the rounded
  // maximum of |s| (range of s)
  uint32_t scale;
  Block<BO> ob;
  uint32_t yw[kBlockValues / 2];  // decoded re-encoded sum as dtype pairs (WITH_Y)
  if constexpr (Format<BO>::kAsym) {
    // range ends from integer maxima of the fp32 patterns (as in quantize_words_asym)
    int hb = 0;
    uint32_t lb = 0;
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) {
      hb = __builtin_elementwise_max(hb, __builtin_bit_cast(int, s[i]));
      lb = __builtin_elementwise_max(lb, __builtin_bit_cast(uint32_t, s[i]));
    }
    hb = group_max_i32(hb);
    lb = group_max_u32(lb);
    const float hi = round_to_dtype<DT>(__builtin_bit_cast(float, hb));
    const float lo = (lb & 0x80000000u) ? round_to_dtype<DT>(__builtin_bit_cast(float, lb)) : 0.0f;
    float d, e, z;
    scale = group_params<BO>(lo, hi, d, e, z);
    const float zb = z - 256.0f;
    uint32_t t[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; i += 2) {
      float v0, v1;
      round_scale2<DT>(s[i], s[i + 1], e, v0, v1);
      t[i] = quantize_asym<BO>(v0, zb);
      t[i + 1] = quantize_asym<BO>(v1, zb);
    }
    if constexpr (WITH_Y) {  // decode of the re-encoded sum, straight from the codes
      if constexpr (DT == kFp16 && QR_Y_HALF_PAIRS) {
        const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)scale);
        const _Float16 nz = -(_Float16)(1024.0f + z);  // exact: 1024 + z < 2048
#pragma unroll
        for (int i = 0; i < kBlockValues; i += 2)
          yw[i / 2] = decode_pair_asym_fp16(t[i], t[i + 1], f16x2{nz, nz}, f16x2{sh, sh});
      } else {
        const float zm = kMagicBase + z;
#pragma unroll
        for (int i = 0; i < kBlockValues; i += 2)
          yw[i / 2] = pack2<DT>(code_value_asym(t[i], zm) * d, code_value_asym(t[i + 1], zm) * d);
      }
    }
    pack_block<BO>(t, ob);
  } else if constexpr (Format<BO>::kFp4) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(s[i]));
    float d, e;
    scale = fp4_block_scale(round_to_dtype<DT>(m), d, e);
    float v[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; i += 2) round_scale2<DT>(s[i], s[i + 1], e, v[i], v[i + 1]);
    pack_block_fp4(v, ob);
    if constexpr (WITH_Y) {  // decode of the re-encoded sum from its codes
      float kk[kBlockValues];
      decode_block_fp4(ob, kk);
#pragma unroll
      for (int i = 0; i < kBlockValues; i += 2) yw[i / 2] = pack2<DT>(kk[i] * d, kk[i + 1] * d);
    }
  } else {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kBlockValues; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(s[i]));
    float d, e;
    scale = block_scale<BO>(round_to_dtype<DT>(m), d, e);
    uint32_t t[kBlockValues];
#pragma unroll
    for (int i = 0; i < kBlockValues; i += 2) {
      float v0, v1;
      round_scale2<DT>(s[i], s[i + 1], e, v0, v1);
      t[i] = quantize<BO>(v0);
      t[i + 1] = quantize<BO>(v1);
    }
    if constexpr (WITH_Y) {  // decode of the re-encoded sum, straight from the codes
      if constexpr (DT == kFp16 && QR_Y_HALF_PAIRS) {
        const _Float16 dh = __builtin_bit_cast(_Float16, (uint16_t)scale);
#pragma unroll
        for (int i = 0; i < kBlockValues; i += 2) yw[i / 2] = decode_pair_fp16<BO>(t[i], t[i + 1], f16x2{dh, dh});
      } else {
#pragma unroll
        for (int i = 0; i < kBlockValues; i += 2)
          yw[i / 2] = pack2<DT>(code_value<BO>(t[i]) * d, code_value<BO>(t[i + 1]) * d);
      }
    }
    pack_block<BO>(t, ob);
  }
  const TileRef otile = tile_ref(a.out + (size_t)tile * TBO, TBO);
  if constexpr (kStaged<BO>) {
    // codes through the LDS staging region first, then the output tile
    stage_codes_out<QR_RED_STORE_POL>(tl, lane, ob, otile);
    store_block<BO, QR_RED_STORE_POL>(otile, lane, ob, scale);
    if constexpr (WITH_Y) write_lane_words(tl, lane, yw);
  } else {
    if constexpr (WITH_Y) write_lane_words(tl, lane, yw);
    store_block<BO, QR_RED_STORE_POL>(otile, lane, ob, scale);
  }
  if constexpr (WITH_Y)
    flush_tile<QR_RED_Y_STORE_POL>(tl, lane, tile_ref(a.y + (size_t)tile * (kTileValues * 2), kTileValues * 2));
}

// Whether every rank's loads are issued before the decode starts: where R
// blocks of codes fit in registers beside the sum and the decode temporaries
// (with 8-bit codes at R = 15 and 16 they would not: the compiler then parks
// registers in AGPRs and the kernel drops to one wave per SIMD).
template <int BI, int R>
constexpr bool kLoadsFirst = QR_RED_LOADS_FIRST && R * (int)(sizeof(Block<BI>) / 4 + 1) <= QR_RED_LOADS_FIRST_REGS;

template <int BI, int BO, int DT, int R, bool WITH_Y, bool ORDER>
__global__ __launch_bounds__(kThreads) void reduce_kernel(ReduceArgs a) {
  static_assert(Format<BI>::kAsym == Format<BO>::kAsym && Format<BI>::kFp4 == Format<BO>::kFp4,
                "a reduce stays within one format family");
  __shared__ u32x4 lds[kWavesPerGroup][kReduceLdsChunks<BI, BO, WITH_Y>];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // uniform per wave
  const int stride = gridDim.x * kWavesPerGroup;
  int tile = group_index<Format<BI>::kTileBytes, Format<BO>::kTileBytes>(blockIdx.x, gridDim.x) * kWavesPerGroup +
             wave;
  if constexpr (QR_RED_PREFETCH) {
    // Each wave loops over several tiles with two register sets: the next
    // tile's loads are in flight while the current tile is reduced.
    if (tile >= a.ntiles) return;
    Block<BI> ba[R], bb[R];
    uint32_t sa[R], sb[R];
    load_ranks<BI, R>(a, tile, lane, ba, sa);
    for (;;) {
      int next = tile + stride;
      const bool more = next < a.ntiles;
      if (more) load_ranks<BI, R>(a, next, lane, bb, sb);
      __builtin_amdgcn_sched_barrier(0);
      reduce_tile<BI, BO, DT, R, WITH_Y, ORDER>(a, tile, lane, lds[wave], ba, sa);
      if (!more) break;
      tile = next;
      next = tile + stride;
      const bool more2 = next < a.ntiles;
      if (more2) load_ranks<BI, R>(a, next, lane, ba, sa);
      __builtin_amdgcn_sched_barrier(0);
      reduce_tile<BI, BO, DT, R, WITH_Y, ORDER>(a, tile, lane, lds[wave], bb, sb);
      if (!more2) break;
      tile = next;
    }
  } else {
    for (; tile < a.ntiles; tile += stride) {
      Block<BI> blk[R];
      uint32_t sc[R];
      if constexpr (Format<BI>::kCodeBits == 3 && QR_INT3_LDS_STAGE) {
        // every rank's tile in one 16-byte load per lane, then handed out
        // through LDS rank by rank before the decode starts
        u32x4 raw[R];
        const size_t toff = (size_t)tile * Format<BI>::kTileBytes;
#pragma unroll
        for (int r = 0; r < R; ++r)
          raw[r] = ld16<QR_RED_LOAD_POL>(tile_ref(a.ranks[r] + toff, Format<BI>::kTileBytes), 16 * lane);
#pragma unroll
        for (int r = 0; r < R; ++r) stage_int3_in(lds[wave], lane, raw[r], blk[r], sc[r]);
      } else {
        load_ranks<BI, R>(a, tile, lane, blk, sc);
        if constexpr (kLoadsFirst<BI, R>) __builtin_amdgcn_sched_barrier(0);
      }
      reduce_tile<BI, BO, DT, R, WITH_Y, ORDER>(a, tile, lane, lds[wave], blk, sc);
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

// Launches a kernel with kThreads threads per workgroup and returns the status
// of that launch itself (hipGetLastError could also report an earlier failure
// of an unrelated call on the same thread).  The parameter types come from the
// kernel alone, so each argument is converted to its parameter's type.
// `lds` bytes of dynamic LDS are allocated per workgroup (the kernels never
// address them: they only limit residency, see residency_pad()).
template <typename... P>
struct Launch {
  void (*kernel)(P...);
  qr_status operator()(dim3 grid, unsigned lds, hipStream_t st, P... args) const {
    void* argv[] = {static_cast<void*>(&args)...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kThreads), argv, lds, st) ==
                   hipSuccess
               ? QR_OK
               : QR_ERR_HIP;
  }
};
template <typename... P>
Launch<P...> launch(void (*kernel)(P...)) {
  return {kernel};
}

// Compute units of the current device (qr_api.hip; 0 if it cannot be queried).
int device_compute_units();

// Dynamic LDS bytes per workgroup that leave room for at most `groups`
// workgroups of a kernel with `static_bytes` of LDS on one CU, or 0 (no cap):
// when `groups` is 0, or the grid of `nwg` workgroups has at most
// QR_CAP_MIN_GROUPS per CU.
inline unsigned residency_pad(unsigned nwg, int static_bytes, int groups) {
  if (groups <= 0) return 0;
  const int cus = device_compute_units();
  if (cus <= 0 || nwg <= (unsigned)cus * QR_CAP_MIN_GROUPS) return 0;
  const int per_group = kLdsBytesPerCU / groups;
  return per_group > static_bytes ? (unsigned)(per_group - static_bytes) : 0u;
}

template <int BITS>
qr_status launch_encode(int dt, const void* x, void* p, size_t ntiles, hipStream_t st) {
  constexpr int kStatic = kWavesPerGroup * kEncLdsChunks * 16;
  if constexpr (QR_ENC_GROUP8 && (BITS == 3 || BITS == 4)) {
    const dim3 grid = grid_for(ntiles);
    auto k = dt == kFp16 ? launch(encode_group8_kernel<BITS, kFp16>) : launch(encode_group8_kernel<BITS, kBf16>);
    return k(grid, residency_pad(grid.x, kStatic, QR_ENC_GROUPS_PER_CU), st, (const uint8_t*)x, (uint8_t*)p,
             (int)ntiles);
  }
  const dim3 grid = grid_for((ntiles + QR_ENC_TILES_PER_WAVE - 1) / QR_ENC_TILES_PER_WAVE);
  auto k = dt == kFp16 ? launch(encode_kernel<BITS, kFp16>) : launch(encode_kernel<BITS, kBf16>);
  return k(grid, residency_pad(grid.x, kStatic, QR_ENC_GROUPS_PER_CU), st, (const uint8_t*)x, (uint8_t*)p,
           (int)ntiles);
}

template <int BITS>
qr_status launch_decode(int dt, const void* p, void* y, size_t ntiles, hipStream_t st) {
  constexpr int kStatic = kWavesPerGroup * kDecLdsChunks * 16;
  const dim3 grid = grid_for(ntiles);
  auto k = dt == kFp16 ? launch(decode_kernel<BITS, kFp16>) : launch(decode_kernel<BITS, kBf16>);
  return k(grid, residency_pad(grid.x, kStatic, QR_DEC_GROUPS_PER_CU_MAX), st, (const uint8_t*)p, (uint8_t*)y,
           (int)ntiles);
}

template <int BI, int BO, int DT, int R, bool ORDER>
qr_status launch_reduce_o(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  constexpr int kCap = kStaged<BI> ? QR_RED8_GROUPS_PER_CU_MAX : QR_RED_GROUPS_PER_CU_MAX;
  if (a.y) {
    constexpr int kStatic = kWavesPerGroup * kReduceLdsChunks<BI, BO, true> * 16;
    return launch(reduce_kernel<BI, BO, DT, R, true, ORDER>)(grid, residency_pad(grid.x, kStatic, kCap), st, a);
  }
  constexpr int kStatic = kWavesPerGroup * kReduceLdsChunks<BI, BO, false> * 16;
  return launch(reduce_kernel<BI, BO, DT, R, false, ORDER>)(grid, residency_pad(grid.x, kStatic, kCap), st, a);
}

template <int BI, int BO, int DT, int R>
qr_status launch_reduce_r(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  if constexpr (kOrderMode<BI> == 2) {
    if (a.ntiles <= QR_RED_ORDER_MAX_TILES) return launch_reduce_o<BI, BO, DT, R, true>(a, grid, st);
    return launch_reduce_o<BI, BO, DT, R, false>(a, grid, st);
  } else {
    return launch_reduce_o<BI, BO, DT, R, kOrderMode<BI> == 1>(a, grid, st);
  }
}

template <int BI, int BO, int DT>
qr_status launch_reduce_dt(const ReduceArgs& a, dim3 grid, hipStream_t st) {
  switch (a.R) {
#define QR_RANK_CASE(r) \
  case r: return launch_reduce_r<BI, BO, DT, r>(a, grid, st);
    QR_RANK_CASE(1) QR_RANK_CASE(2) QR_RANK_CASE(3) QR_RANK_CASE(4)
    QR_RANK_CASE(5) QR_RANK_CASE(6) QR_RANK_CASE(7) QR_RANK_CASE(8)
    QR_RANK_CASE(9) QR_RANK_CASE(10) QR_RANK_CASE(11) QR_RANK_CASE(12)
    QR_RANK_CASE(13) QR_RANK_CASE(14) QR_RANK_CASE(15) QR_RANK_CASE(16)
#undef QR_RANK_CASE
    default: return QR_ERR_ARG;  // R is validated to be in [1, QR_MAX_RANKS] before this
  }
}

// Reduce grid: one wave per tile, or with QR_RED_PREFETCH at most
// QR_RED_GROUPS_PER_CU workgroups per compute unit, each wave looping.
inline dim3 reduce_grid(size_t ntiles) {
  dim3 g = grid_for(ntiles);
  if constexpr (QR_RED_PREFETCH) {
    const int cus = device_compute_units();
    if (cus > 0 && g.x > (unsigned)(cus * QR_RED_GROUPS_PER_CU)) g.x = (unsigned)(cus * QR_RED_GROUPS_PER_CU);
  }
  return g;
}

template <int BI, int BO>
qr_status launch_reduce(int dt, const ReduceArgs& a, hipStream_t st) {
  const dim3 grid = reduce_grid((size_t)a.ntiles);
  return dt == kFp16 ? launch_reduce_dt<BI, BO, kFp16>(a, grid, st) : launch_reduce_dt<BI, BO, kBf16>(a, grid, st);
}

// Reduce with input format != output format (instantiated in qr_reduce_mixed.hip,
// one object per input format).
qr_status launch_reduce_mixed_from3(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
qr_status launch_reduce_mixed_from4(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
qr_status launch_reduce_mixed_from8(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
// Asymmetric formats (qr_asym.hip, one object per input format): encode,
// decode and the reduce into either asymmetric output format.
qr_status launch_encode_asym(int fmt, int dt, const void* x, void* p, size_t ntiles, hipStream_t st);
qr_status launch_decode_asym(int fmt, int dt, const void* p, void* y, size_t ntiles, hipStream_t st);
qr_status launch_reduce_asym_from20(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
qr_status launch_reduce_asym_from24(int fmt_out, int dt, const ReduceArgs& a, hipStream_t st);
// FP4 E2M1 format (qr_fp4.hip): encode, decode and the same-format reduce.
qr_status launch_encode_fp4(int dt, const void* x, void* p, size_t ntiles, hipStream_t st);
qr_status launch_decode_fp4(int dt, const void* p, void* y, size_t ntiles, hipStream_t st);
qr_status launch_reduce_fp4(int dt, const ReduceArgs& a, hipStream_t st);

}  // namespace qr
