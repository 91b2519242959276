// qr_codec.hpp -- gfx950 device code of the 32-value block codec.
//
// Format ("QuickReduce INT3 quantization and benchmarking on MI355", section
// "Design Highlights"; INT8 extends the same block framework to 8 bits):
//   block  = 32 consecutive values, one fp16 scale d = fp16(min(max|x|/Q, 65504))
//   code   = clamp(round_half_even(x * e), -Q, Q-1) + Q, e = fp32(1/d) (0 if d == 0)
//   INT4   word u = unit of 8 values, value j at bits 4j (lowest first, as the
//          packed int32 nibbles of vLLM PR #54965 / PR #43389)
//   INT3   2-bit plane (uint16 per unit, value j at bits 2j) + 1-bit plane
//          (uint8 per unit, value j at bit j)
//   decode = (code - Q) * d, exact in fp32.
// Asymmetric group codec (the "Flash Communication" review of arXiv
// 2412.04964, fields pith_summary / key_machinery: group size 128, a scale and
// a zero point per group; minor_comments on Algorithm 1: (q - z) * s):
//   group  = 128 consecutive values, range [lo, hi] = [min(x, 0), max(x, 0)]
//   scale  s = fp16(min((hi - lo) / (2^b - 1), 65504)), e = fp32(1/s) (0 if s == 0)
//   zero   z = clamp(rint(-lo * e), 0, 2^b - 1), one byte per group
//   code   q = clamp(rint(x * e) + z, 0, 2^b - 1), packed as the INT4 / INT8 codes
//   decode = (q - z) * s, exact in fp32.
// FP4 block codec (OCP MX E2M1 elements in the INT4 framework; the
// QuickReduce MI355 blog's introduction names a hardware FP4 path there):
//   scale  d = fp16(min(max|x| / 6, 65504)), e = fp32(1/d) (0 if d == 0)
//   code   = the E2M1 value nearest to x * e (ties to even, saturating, sign
//          kept), by the gfx950 scaled FP4 conversion with scale 1.0
//   decode = value * d, exact in fp32.
//
// Work mapping: one lane owns one block (32 values), one 64-lane wave owns one
// 2048-value tile; a 128-value asymmetric group is four lanes (DPP quad
// permutes).  The block maximum and the scale are computed once per lane; the
// fp16/bf16 side of a tile, and 8-bit codes, move through wave-private LDS so
// that every global access is a coalesced 16-byte access.  Nothing here is a
// contraction, so there is no MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileValues = 2048;
constexpr int kBlockValues = 32;
constexpr int kWave = 64;
constexpr int kChunks = kTileValues * 2 / 16;  // 16-byte chunks of one fp16/bf16 tile

enum { kFp16 = 0, kBf16 = 1 };

// Formats are named by their qr_format value: 3, 4, 8 (symmetric, 32-value
// blocks), 20, 24 (asymmetric, 128-value groups, 4- and 8-bit codes) and 36
// (FP4 E2M1 codes in 32-value blocks).
template <int F>
struct Format;
// 1: the reduce loads each INT3 rank tile with one 16-byte load per lane and
// hands the blocks out through LDS (stage_int3_in()); 0: each lane loads its
// own block's planes and scale (8 + 4 + 2 bytes).  Measured slower; kept for
// comparison.
#ifndef QR_INT3_LDS_STAGE
#define QR_INT3_LDS_STAGE 0
#endif

// 1: INT3 codes decode through a byte table (one permute maps four 3-bit
// codes to the FP8 E4M3 values of code - 4, one conversion turns two of them
// into fp32); 0: through signed bytes 32 * (code - 4).
#ifndef QR_INT3_TABLE_DECODE
#define QR_INT3_TABLE_DECODE 1
#endif

template <>
struct Format<3> {
  static constexpr bool kAsym = false;
  static constexpr bool kFp4 = false;
  static constexpr int kCodeBits = 3;
  static constexpr int kQ = 4;
  static constexpr int kTileBytes = 896;   // 512 (2-bit plane) + 256 (1-bit plane) + 128
  static constexpr int kScaleOffset = 768;
  static constexpr int kHighOffset = 512;  // the 1-bit plane
  static constexpr int kShift = QR_INT3_TABLE_DECODE ? 0 : 5;  // decoded values are 2^kShift * k
};
template <>
struct Format<4> {
  static constexpr bool kAsym = false;
  static constexpr bool kFp4 = false;
  static constexpr int kCodeBits = 4;
  static constexpr int kQ = 8;
  static constexpr int kTileBytes = 1152;  // 1024 + 128
  static constexpr int kScaleOffset = 1024;
  static constexpr int kShift = 4;         // decoded bytes hold 16 * k
};
template <>
struct Format<8> {
  static constexpr bool kAsym = false;
  static constexpr bool kFp4 = false;
  static constexpr int kCodeBits = 8;
  static constexpr int kQ = 128;
  static constexpr int kTileBytes = 2176;  // 2048 + 128
  static constexpr int kScaleOffset = 2048;
  static constexpr int kShift = 0;
};
template <>
struct Format<20> {
  static constexpr bool kAsym = true;
  static constexpr bool kFp4 = false;
  static constexpr int kCodeBits = 4;
  static constexpr int kQmax = 15;
  static constexpr int kTileBytes = 1072;  // 1024 codes + 16 fp16 scales + 16 zero points
  static constexpr int kScaleOffset = 1024;
  static constexpr int kZeroOffset = 1056;
  static constexpr int kShift = 0;
  static constexpr int kOddShift = 4;  // odd values decode as 16 (q - z)
};
template <>
struct Format<24> {
  static constexpr bool kAsym = true;
  static constexpr bool kFp4 = false;
  static constexpr int kCodeBits = 8;
  static constexpr int kQmax = 255;
  static constexpr int kTileBytes = 2096;  // 2048 codes + 16 fp16 scales + 16 zero points
  static constexpr int kScaleOffset = 2048;
  static constexpr int kZeroOffset = 2080;
  static constexpr int kShift = 0;
  static constexpr int kOddShift = 0;
};

// FP4: OCP MX E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa
// bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6) in INT4's block framework.
template <>
struct Format<36> {
  static constexpr bool kAsym = false;
  static constexpr bool kFp4 = true;
  static constexpr int kCodeBits = 4;
  static constexpr int kTileBytes = 1152;  // 1024 + 128, as INT4
  static constexpr int kScaleOffset = 1024;
  static constexpr int kShift = 0;
};

// Packed codes of one 32-value block as held by its lane, by code width.
template <int CB>
struct CodeBlock;
template <>
struct CodeBlock<4> {
  uint32_t w[4];  // units 0..3
};
template <>
struct CodeBlock<3> {
  uint32_t low[2];  // 2-bit plane: units 0,1 in low[0] (unit 0 in bits 0..15), units 2,3 in low[1]
  uint32_t high;    // 1-bit plane: byte u = unit u
};
template <>
struct CodeBlock<8> {
  uint32_t w[8];  // byte i of the block = value i
};
template <int F>
using Block = CodeBlock<Format<F>::kCodeBits>;

// ---------------------------------------------------------------------------
// dtype <-> fp32
// ---------------------------------------------------------------------------

template <int DT>
__device__ __forceinline__ float lo_to_f32(uint32_t w) {
  if constexpr (DT == kFp16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
  else
    return __builtin_bit_cast(float, w << 16);
}

template <int DT>
__device__ __forceinline__ float hi_to_f32(uint32_t w) {
  if constexpr (DT == kFp16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  else
    return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Two fp32 values to a packed dtype pair (low half first), round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  f32x2 v = {a, b};
  if constexpr (DT == kFp16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The dtype value nearest to s (ties to even), as fp32.
template <int DT>
__device__ __forceinline__ float round_to_dtype(float s) {
  if constexpr (DT == kFp16)
    return (float)(_Float16)s;
  else
    return (float)(__bf16)s;
}

// -0.0f in a VGPR the optimizer cannot see through: fma(x, e, -0) is exactly
// the IEEE product x*e, but folded to a multiply it would need a separate
// fp16 -> fp32 conversion instead of one mixed-precision FMA.
__device__ __forceinline__ float opaque_neg_zero() {
  float z = -0.0f;
  asm("" : "+v"(z));
  return z;
}

// RN32(dtype_RNE(s) * e) for two values at once: one packed conversion to the
// dtype, then for fp16 a mixed-precision FMA that reads the fp16 halves
// directly.  fma(z, e, -0) is exactly the IEEE product z*e, the sign of a zero
// included (the FP4 codes keep it).
template <int DT>
__device__ __forceinline__ void round_scale2(float s0, float s1, float e, float& v0, float& v1) {
  f32x2 s = {s0, s1};
  if constexpr (DT == kFp16) {
    const f16x2 h = __builtin_convertvector(s, f16x2);
    const float nz = opaque_neg_zero();
    v0 = __builtin_fmaf((float)h.x, e, nz);
    v1 = __builtin_fmaf((float)h.y, e, nz);
  } else {
    const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(s, bf16x2));
    v0 = __builtin_bit_cast(float, b << 16) * e;
    v1 = __builtin_bit_cast(float, b & 0xffff0000u) * e;
  }
}

// A 32-bit constant held in a VGPR, so that a three-operand bit operation can
// take it together with a second constant (one scalar operand per VOP3).
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}

// Signed byte i of x as fp32 (one SDWA conversion on gfx950).
__device__ __forceinline__ float sbyte(uint32_t x, int i) { return (float)(int8_t)(x >> (8 * i)); }

// ---------------------------------------------------------------------------
// wave-private LDS tile: 256 chunks of 16 bytes, stored with one 16-byte pad
// after every 16 chunks (272 slots): chunk c lives in slot c + c / 16.  Both
// access orders are then a per-lane base plus a constant (the instruction's
// immediate offset, so the addresses are computed once per wave):
//   row order   (lane L, chunks L + 64k): slot L + L / 16 + 68k
//   block order (lane l, chunks 4l + j):  slot 4l + l / 4 + j
// and the 16 lanes of every aligned group of 16 hit 16 distinct slots modulo
// 16 (distinct 16-byte bank groups of a 64-bank LDS) in both orders.
// ---------------------------------------------------------------------------

constexpr int kTileSlots = kChunks + kChunks / 16;

__device__ __forceinline__ uint32_t row_slot(uint32_t lane, int k) { return lane + (lane >> 4) + 68 * k; }
__device__ __forceinline__ uint32_t block_slot(uint32_t lane, int j) { return 4 * lane + (lane >> 2) + j; }

// Makes one lane's LDS writes visible to the other lanes of its wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// packing of codes (code in the low byte of each word of c[])
// ---------------------------------------------------------------------------

// bytes [a.b0, b.b0, 0, 0] and [0, 0, a.b0, b.b0]
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x0c0c0400u);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x04000c0cu);
}

// INT4 word of one unit: value j at bits 4j.
__device__ __forceinline__ uint32_t pack_int4_unit(const uint32_t* c) {
  uint32_t even = lo_pair(c[0], c[2]) | hi_pair(c[4], c[6]);  // bytes c0 c2 c4 c6
  uint32_t odd = lo_pair(c[1], c[3]) | hi_pair(c[5], c[7]);   // bytes c1 c3 c5 c7
  return even | (odd << 4);
}

// INT8 word: bytes c0 c1 c2 c3.
__device__ __forceinline__ uint32_t pack_int8_word(const uint32_t* c) {
  return lo_pair(c[0], c[1]) | hi_pair(c[2], c[3]);
}

__device__ __forceinline__ uint32_t bit_select(uint32_t mask, uint32_t a, uint32_t b) {
  return (a & mask) | (b & ~mask);  // v_bfi_b32
}

// INT3 planes of 16 values (two units): the 2-bit plane dword (unit 0 in the
// low 16 bits) and a word whose bytes 0 and 2 are the two 1-bit plane bytes.
__device__ __forceinline__ void pack_int3_pair(const uint32_t* c, uint32_t& low, uint32_t& highx) {
  uint32_t g[4];  // g[r] byte b = code of value 4b + r
#pragma unroll
  for (int r = 0; r < 4; ++r) g[r] = lo_pair(c[r], c[4 + r]) | hi_pair(c[8 + r], c[12 + r]);
  // byte b of `low` = low pairs of values 4b..4b+3 at bits 0,2,4,6
  uint32_t y = bit_select(0xC0C0C0C0u, g[3] << 6, g[2] << 4);
  y = bit_select(0xF0F0F0F0u, y, g[1] << 2);
  low = bit_select(0xFCFCFCFCu, y, g[0]);
  // byte b bits 0..3 of `s` = high bits of values 4b..4b+3
  uint32_t s = (g[0] >> 2) & 0x01010101u;
  s = bit_select(0x02020202u, g[1] >> 1, s);
  s = bit_select(0x04040404u, g[2], s);
  s = bit_select(0x08080808u, g[3] << 1, s);
  highx = s | (s >> 4);
}

// ---------------------------------------------------------------------------
// one block: encode (from exact dtype values in fp32) and decode
// ---------------------------------------------------------------------------

// Magic constant 2^23 + 0x6400 + Q: adding it to a value in [-Q, Q) rounds
// that value to an integer (half to even: the sum lies in [2^23, 2^24), where
// the fp32 spacing is 1) and leaves the biased code q = k + Q in the low byte
// of the mantissa, with 0x64 in the byte above it:
// bits(2^23 + 0x6400 + Q + k) = 0x4B006400 + q.  The low two bytes are then
// the fp16 pattern of 1024 + q, so one byte permute makes an fp16 pair of
// codes (used by the fused decode of the re-encoded sum).
constexpr float kMagicBase = 8388608.0f + 25600.0f;  // 2^23 + 0x6400
template <int BITS>
__device__ __forceinline__ constexpr float magic() {
  return kMagicBase + Format<BITS>::kQ;
}

// fp32(1 / d), correctly rounded, for d a positive finite fp16 value: the
// hardware reciprocal estimate followed by one Newton step r + r * (1 - d * r)
// (both FMAs single-rounded).  Exhaustively equal to the IEEE quotient 1.0f / d
// over all 31743 positive finite fp16 values on gfx950 (the estimate alone is
// off by an ulp for 2746 of them); three instructions instead of the eleven of
// the general correctly rounded division.
__device__ __forceinline__ float recip_fp16_value(float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  return __builtin_fmaf(r, __builtin_fmaf(-d, r, 1.0f), r);
}

// Scale of a block from its absolute maximum m: d = fp16(min(m / Q, 65504))
// (m / Q is exact).  Returns the fp16 bits; d and the encode multiplier
// e = fp32(1 / d) (0 when d == 0) are set.
template <int BITS>
__device__ __forceinline__ uint32_t block_scale(float m, float& d, float& e) {
  constexpr int Q = Format<BITS>::kQ;
  const _Float16 dh = (_Float16)__builtin_fminf(m * (1.0f / Q), 65504.0f);
  d = (float)dh;
  e = (d == 0.0f) ? 0.0f : recip_fp16_value(d);
  return __builtin_bit_cast(uint16_t, dh);
}

// Code of one value: q = clamp(rint(RN32(x * e)), -Q, Q-1) + Q, returned as
// the bits of 2^23 + 0x6400 + q (low byte = q).  Clamping after the magic add
// equals clamping before rounding because the bounds are integers.
template <int BITS>
__device__ __forceinline__ uint32_t quantize(float v) {
  constexpr int Q = Format<BITS>::kQ;
  const float t = __builtin_amdgcn_fmed3f(v + magic<BITS>(), kMagicBase, kMagicBase + (2 * Q - 1));
  return __builtin_bit_cast(uint32_t, t);
}

// code - Q as fp32 from quantize()'s result (exact).
template <int BITS>
__device__ __forceinline__ float code_value(uint32_t t) {
  return __builtin_bit_cast(float, t) - magic<BITS>();
}

// fp16 pair dtype_RNE((q0 - Q) * d), dtype_RNE((q1 - Q) * d) from two
// quantize() results and the fp16 scale d: one byte permute gives the fp16
// pair (1024 + q0, 1024 + q1), one packed subtract the exact codes q - Q, and
// one packed multiply the products, each rounded once to fp16 (the exact
// product has at most 8 + 11 significant bits, so this equals rounding the
// exact fp32 product, overflow to infinity included).
template <int BITS>
__device__ __forceinline__ uint32_t decode_pair_fp16(uint32_t t0, uint32_t t1, f16x2 d2) {
  constexpr _Float16 kBias = (_Float16)(-(1024 + Format<BITS>::kQ));
  const f16x2 k = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(t1, t0, 0x05040100u)) + f16x2{kBias, kBias};
  return __builtin_bit_cast(uint32_t, k * d2);
}

// Packs 32 codes (low byte of each t[i]) into the lane's block.
template <int F>
__device__ __forceinline__ void pack_block(const uint32_t (&t)[kBlockValues], Block<F>& blk) {
  constexpr int BITS = Format<F>::kCodeBits;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) blk.w[u] = pack_int4_unit(t + 8 * u);
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int w = 0; w < 8; ++w) blk.w[w] = pack_int8_word(t + 4 * w);
  } else {
    uint32_t h0, h1;
    pack_int3_pair(t, blk.low[0], h0);
    pack_int3_pair(t + 16, blk.low[1], h1);
    blk.high = __builtin_amdgcn_perm(h1, h0, 0x06040200u);
  }
}

// Largest |x| of a block held as 16 packed fp16/bf16 words, as fp32: the
// sign bits are cleared and the magnitudes compared as unsigned 16-bit
// integers, which orders non-negative fp16 / bf16 values (inputs are finite).
template <int DT>
__device__ __forceinline__ float block_absmax(const uint32_t (&w)[kBlockValues / 2]) {
  u16x2 m = {0, 0};
#pragma unroll
  for (int j = 0; j < kBlockValues / 2; ++j)
    m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[j] & 0x7fff7fffu));
  const uint32_t mb = m.x > m.y ? m.x : m.y;
  if constexpr (DT == kFp16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)mb);
  else
    return __builtin_bit_cast(float, mb << 16);
}

// RN32(x * e) for the two values of a packed fp16/bf16 word (for fp16 a
// mixed-precision FMA reads the halves directly; fma(x, e, -0) is exactly the
// IEEE product x*e, the sign of a zero included).
template <int DT>
__device__ __forceinline__ void scale_pair(uint32_t w, float e, float& v0, float& v1) {
  if constexpr (DT == kFp16) {
    const f16x2 h = __builtin_bit_cast(f16x2, w);
    const float nz = opaque_neg_zero();
    v0 = __builtin_fmaf((float)h.x, e, nz);
    v1 = __builtin_fmaf((float)h.y, e, nz);
  } else {
    v0 = __builtin_bit_cast(float, w << 16) * e;
    v1 = __builtin_bit_cast(float, w & 0xffff0000u) * e;
  }
}

// Quantizes one block given as 16 packed fp16/bf16 words (value 2j in the low
// half of word j) into t[] (see quantize()); returns the fp16 scale bits.
template <int BITS, int DT>
__device__ __forceinline__ uint32_t quantize_words(const uint32_t (&w)[kBlockValues / 2],
                                                   uint32_t (&t)[kBlockValues]) {
  float d, e;
  const uint32_t bits = block_scale<BITS>(block_absmax<DT>(w), d, e);
#pragma unroll
  for (int j = 0; j < kBlockValues / 2; ++j) {
    float v0, v1;
    scale_pair<DT>(w[j], e, v0, v1);
    t[2 * j] = quantize<BITS>(v0);
    t[2 * j + 1] = quantize<BITS>(v1);
  }
  return bits;
}

// Decodes one block into kk[i] = 2^Format::kShift * (code_i - Q) as fp32.
// The value is kk[i] * (d * 2^-kShift), an exact product.
template <int F>
__device__ __forceinline__ void decode_block(const Block<F>& blk, float (&kk)[kBlockValues]) {
  constexpr int BITS = Format<F>::kCodeBits;
  static_assert(!Format<F>::kAsym, "asymmetric formats decode with decode_block_asym");
  if constexpr (BITS == 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // high nibble of each byte, top bit flipped: 16 * (code - 8) as int8
      const uint32_t hi = (blk.w[u] & 0xF0F0F0F0u) ^ 0x80808080u;         // odd values
      const uint32_t lo = ((blk.w[u] << 4) & 0xF0F0F0F0u) ^ 0x80808080u;  // even values
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kk[8 * u + 2 * i] = sbyte(lo, i);
        kk[8 * u + 2 * i + 1] = sbyte(hi, i);
      }
    }
  } else if constexpr (BITS == 8) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t a = blk.w[w] ^ 0x80808080u;  // byte = code - 128
#pragma unroll
      for (int i = 0; i < 4; ++i) kk[4 * w + i] = sbyte(a, i);
    }
  } else if constexpr (QR_INT3_TABLE_DECODE) {
    // Values 8u + j (u = unit 0..3) are decoded together for each j: two byte
    // gathers give, per unit, the low-pair byte that holds value j; byte u of
    // the 1-bit plane word holds unit u's high bits.  Byte u of `sel` is the
    // code of value 8u + j (low pair | high bit << 2), a permute selector
    // into the table of the FP8 E4M3 bytes of code - 4, and each conversion
    // turns two table bytes into fp32 (exact: the values are -4 .. 3).
    const uint32_t p03 = __builtin_amdgcn_perm(blk.low[1], blk.low[0], 0x06040200u);  // j = 0..3
    const uint32_t p47 = __builtin_amdgcn_perm(blk.low[1], blk.low[0], 0x07050301u);  // j = 4..7
    const uint32_t table_hi = vgpr_const(0x44403800u);  // codes 7..4: 3, 2, 1, 0
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t p = j < 4 ? p03 : p47;
      const int i = j & 3;  // the low pair sits at bits 2i..2i+1 of each byte
      const uint32_t lo = i ? p >> (2 * i) : p;
      const uint32_t hi = j < 2 ? blk.high << (2 - j) : blk.high >> (j - 2);
      const uint32_t sel = (lo & 0x03030303u) | (hi & 0x04040404u);
      const uint32_t t = __builtin_amdgcn_perm(table_hi, 0xB8C0C4C8u, sel);  // codes 3..0: -1 .. -4
      const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 1.0f, false);
      const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(t, 1.0f, true);
      kk[j] = a.x;
      kk[8 + j] = a.y;
      kk[16 + j] = b.x;
      kk[24 + j] = b.y;
    }
  } else {
    // Values 8u + j (u = unit 0..3) are decoded together for each j: byte u
    // of the 1-bit plane word holds unit u's high bits, so one shift puts all
    // four (inverted: the sign of code - 4) at bit 7 of their bytes, and two
    // byte gathers give, per unit, the low-pair byte that holds value j.
    const uint32_t ne = ~blk.high;
    const uint32_t p03 = __builtin_amdgcn_perm(blk.low[1], blk.low[0], 0x06040200u);  // j = 0..3
    const uint32_t p47 = __builtin_amdgcn_perm(blk.low[1], blk.low[0], 0x07050301u);  // j = 4..7
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t p = j < 4 ? p03 : p47;
      const int i = j & 3;  // the low pair sits at bits 2i..2i+1 of each byte
      const uint32_t l = (i < 3 ? (p << (5 - 2 * i)) : (p >> 1)) & 0x60606060u;
      // byte u = (low pair << 5) | (!high << 7) = 32 * (code - 4) as int8
      const uint32_t b = l | ((ne << (7 - j)) & 0x80808080u);
#pragma unroll
      for (int u = 0; u < 4; ++u) kk[8 * u + j] = sbyte(b, u);
    }
  }
}

// ---------------------------------------------------------------------------
// FP4 E2M1 block codec, with the gfx950 scaled FP4 conversions ("QuickReduce
// INT3 quantization and benchmarking on MI355", introduction: a hardware
// FP4 path interchangeable with INT4).  The scale operand of the conversions
// is 1.0: the block scale is applied in fp32 beforehand (encode) or
// afterwards (decode), so every rounding is the one the codec defines.
// ---------------------------------------------------------------------------

// Scale of a block with absolute maximum m (the maximum maps to 6):
// d = fp16(min(m / 6, 65504)), e = fp32(1 / d) (0 if d == 0).  m * fp32(1/6)
// differs from the correctly rounded m / 6 by at most one fp32 ulp and gives
// the same fp16 d for every fp16 and bf16 m (checked exhaustively), so the
// multiply stands in for the division.
__device__ __forceinline__ uint32_t fp4_block_scale(float m, float& d, float& e) {
  const _Float16 dh = (_Float16)__builtin_fminf(m * (1.0f / 6.0f), 65504.0f);
  d = (float)dh;
  e = (d == 0.0f) ? 0.0f : recip_fp16_value(d);
  return __builtin_bit_cast(uint16_t, dh);
}

// E2M1 codes of a and b (nearest, ties to even, saturating at +-6, sign kept)
// into byte SEL of `old`: a in the low nibble, b in the high nibble.
template <int SEL>
__device__ __forceinline__ uint32_t fp4_pack(uint32_t old, float a, float b) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// E2M1 values of the low and high nibble of byte SEL of w.
template <int SEL>
__device__ __forceinline__ f32x2 fp4_unpack(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// Encodes one block given as 16 packed fp16/bf16 words into E2M1 unit words
// (value j of a unit at bits 4j, as INT4).  Returns the fp16 scale bits.
template <int DT>
__device__ __forceinline__ uint32_t quantize_words_fp4(const uint32_t (&w)[kBlockValues / 2], CodeBlock<4>& blk) {
  float d, e;
  const uint32_t bits = fp4_block_scale(block_absmax<DT>(w), d, e);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) scale_pair<DT>(w[4 * u + j], e, v[2 * j], v[2 * j + 1]);
    uint32_t r = fp4_pack<0>(0u, v[0], v[1]);
    r = fp4_pack<1>(r, v[2], v[3]);
    r = fp4_pack<2>(r, v[4], v[5]);
    blk.w[u] = fp4_pack<3>(r, v[6], v[7]);
  }
  return bits;
}

// E2M1 unit words of 32 fp32 values v (already multiplied by the encode multiplier).
__device__ __forceinline__ void pack_block_fp4(const float (&v)[kBlockValues], CodeBlock<4>& blk) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint32_t r = fp4_pack<0>(0u, v[8 * u], v[8 * u + 1]);
    r = fp4_pack<1>(r, v[8 * u + 2], v[8 * u + 3]);
    r = fp4_pack<2>(r, v[8 * u + 4], v[8 * u + 5]);
    blk.w[u] = fp4_pack<3>(r, v[8 * u + 6], v[8 * u + 7]);
  }
}

// Decodes one block into kk[i] = the E2M1 value of code i (exact; times the
// block scale it is the decoded value, also exact).
__device__ __forceinline__ void decode_block_fp4(const CodeBlock<4>& blk, float (&kk)[kBlockValues]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const f32x2 p0 = fp4_unpack<0>(blk.w[u]), p1 = fp4_unpack<1>(blk.w[u]);
    const f32x2 p2 = fp4_unpack<2>(blk.w[u]), p3 = fp4_unpack<3>(blk.w[u]);
    kk[8 * u + 0] = p0.x; kk[8 * u + 1] = p0.y; kk[8 * u + 2] = p1.x; kk[8 * u + 3] = p1.y;
    kk[8 * u + 4] = p2.x; kk[8 * u + 5] = p2.y; kk[8 * u + 6] = p3.x; kk[8 * u + 7] = p3.y;
  }
}

// ---------------------------------------------------------------------------
// asymmetric group codec: a group of 128 values is the blocks of four
// consecutive lanes (lanes 4g..4g+3 of a wave hold group g of its tile)
// ---------------------------------------------------------------------------

// Maximum over the four lanes of a group (DPP quad permutes [1,0,3,2] and
// [2,3,0,1]; every lane of the wave is active).
template <int CTRL>
__device__ __forceinline__ int quad_perm(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int group_max_i32(int v) {
  v = __builtin_elementwise_max(v, quad_perm<0xB1>(v));
  return __builtin_elementwise_max(v, quad_perm<0x4E>(v));
}
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  v = __builtin_elementwise_max(v, (uint32_t)quad_perm<0xB1>((int)v));
  return __builtin_elementwise_max(v, (uint32_t)quad_perm<0x4E>((int)v));
}

// fp32 value of an fp16 / bf16 bit pattern held in the low 16 bits.
template <int DT>
__device__ __forceinline__ float half_pattern_to_f32(uint32_t h) {
  if constexpr (DT == kFp16)
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  else
    return __builtin_bit_cast(float, h << 16);
}

// Scale, multiplier and zero point of a group with range [lo, hi], lo <= 0 <= hi:
// s = fp16(min(RN32(RN32(hi - lo) / qmax), 65504)) (a correctly rounded fp32
// division), e = fp32(1 / s) (0 if s == 0), z = clamp(rint(RN32(-lo * e)), 0, qmax).
// Returns s's bits | z << 16.
template <int F>
__device__ __forceinline__ uint32_t group_params(float lo, float hi, float& d, float& e, float& z) {
  constexpr float kQmax = (float)Format<F>::kQmax;
  const float t = (hi - lo) / kQmax;
  const _Float16 dh = (_Float16)__builtin_fminf(t, 65504.0f);
  d = (float)dh;
  e = (d == 0.0f) ? 0.0f : recip_fp16_value(d);
  z = __builtin_amdgcn_fmed3f(__builtin_rintf(-lo * e), 0.0f, kQmax);
  return (uint32_t)__builtin_bit_cast(uint16_t, dh) | ((uint32_t)z << 16);
}

// Code of one value, q = clamp(rint(v) + z, 0, qmax), as the bits of
// B + q with B = 2^23 + 0x6400 (low byte = q, 0x64 above it, as quantize());
// zb = z - 256.  Adding B + 256 (even) rounds v to an integer with ties to
// even for every v >= -(0x6400 + 256); adding z first would move ties for
// odd z.  Smaller v, and large v, land outside [B, B + qmax] and clamp to the
// ends, as the clamp of rint(v) + z does.
template <int F>
__device__ __forceinline__ uint32_t quantize_asym(float v, float zb) {
  const float r = v + (kMagicBase + 256.0f);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_fmed3f(r + zb, kMagicBase, kMagicBase + Format<F>::kQmax));
}

// (q - z) as fp32 from quantize_asym()'s result; zm = B + z (exact).
__device__ __forceinline__ float code_value_asym(uint32_t t, float zm) {
  return __builtin_bit_cast(float, t) - zm;
}

// fp16 pair dtype_RNE((q0 - z) * s), dtype_RNE((q1 - z) * s) from two
// quantize_asym() results, the zero point z and the fp16 scale s (as
// decode_pair_fp16: the exact code difference times s, rounded once).
__device__ __forceinline__ uint32_t decode_pair_asym_fp16(uint32_t t0, uint32_t t1, f16x2 nzb, f16x2 s2) {
  const f16x2 k = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(t1, t0, 0x05040100u)) + nzb;
  return __builtin_bit_cast(uint32_t, k * s2);
}

// Quantizes one lane's block of a group given as 16 packed fp16/bf16 words;
// the four lanes of the group share the range.  Returns scale bits | z << 16.
// The range ends come from two integer maxima of the sign-magnitude bit
// patterns, with no float compares: hi = max(x, 0) is the signed maximum of
// the patterns and 0 (every negative pattern is a negative integer), and the
// unsigned maximum is the negative value of largest magnitude when there is
// one (sign bit set), else non-negative (then min(x, 0) = 0).  Inputs are finite.
template <int F, int DT>
__device__ __forceinline__ uint32_t quantize_words_asym(const uint32_t (&w)[kBlockValues / 2],
                                                        uint32_t (&t)[kBlockValues]) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  s16x2 smax = {0, 0};
  u16x2 umax = {0, 0};
#pragma unroll
  for (int j = 0; j < kBlockValues / 2; ++j) {
    smax = __builtin_elementwise_max(smax, __builtin_bit_cast(s16x2, w[j]));
    umax = __builtin_elementwise_max(umax, __builtin_bit_cast(u16x2, w[j]));
  }
  const int hb = group_max_i32(smax.x > smax.y ? smax.x : smax.y);
  const uint32_t lb = group_max_u32(umax.x > umax.y ? umax.x : umax.y);
  const float hi = half_pattern_to_f32<DT>((uint32_t)hb);
  const float lo = (lb & 0x8000u) ? half_pattern_to_f32<DT>(lb) : 0.0f;
  float d, e, z;
  const uint32_t params = group_params<F>(lo, hi, d, e, z);
  const float zb = z - 256.0f;
#pragma unroll
  for (int j = 0; j < kBlockValues / 2; ++j) {
    float v0, v1;
    scale_pair<DT>(w[j], e, v0, v1);
    t[2 * j] = quantize_asym<F>(v0, zb);
    t[2 * j + 1] = quantize_asym<F>(v1, zb);
  }
  return params;
}

// Decodes one block of an asymmetric format into kk[i] = (q_i - z) * 2^(kOddShift
// * (i & 1)), exactly; odd values then take the scale s * 2^-kOddShift.
// The fp16 pattern 0x6400 | c is the value 1024 + c (c < 1024), so one
// packed fp16 subtract gives two decoded codes at once, exactly (integers
// below 2048), and the fp16 halves feed mixed-precision FMAs directly.
//   4-bit: a unit word holds value j at bits 4j; masking 0x000F000F leaves
//          values 0 and 4 as 1024 + q, masking 0x00F000F0 leaves values 1
//          and 5 as 1024 + 16q (minus 1024 + 16z: 16(q - z)); the word
//          shifted right by 8 gives values 2, 6 and 3, 7 the same way.
//   8-bit: byte gathers put codes 0, 2 and 1, 3 of a word under a 0x64 byte.
// nz and nzo are the fp16 pairs -(1024 + z) and -(1024 + 16 z) (AsymMeta).
template <int F>
__device__ __forceinline__ void decode_block_asym(const Block<F>& blk, f16x2 nz, f16x2 nzo,
                                                  float (&kk)[kBlockValues]) {
  if constexpr (Format<F>::kCodeBits == 4) {
    const uint32_t m0 = vgpr_const(0x000F000Fu), m1 = vgpr_const(0x00F000F0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t src = k < 2 ? blk.w[u] : blk.w[u] >> 8;
        const uint32_t pat = (src & ((k & 1) ? m1 : m0)) | 0x64006400u;
        const f16x2 h = __builtin_bit_cast(f16x2, pat) + ((k & 1) ? nzo : nz);
        kk[8 * u + k] = (float)h.x;
        kk[8 * u + k + 4] = (float)h.y;
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const f16x2 ev = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, blk.w[w], 0x04020400u)) + nz;
      const f16x2 od = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, blk.w[w], 0x04030401u)) + nz;
      kk[4 * w + 0] = (float)ev.x;
      kk[4 * w + 1] = (float)od.x;
      kk[4 * w + 2] = (float)ev.y;
      kk[4 * w + 3] = (float)od.y;
    }
  }
}

// ---------------------------------------------------------------------------
// global <-> lane block data
// ---------------------------------------------------------------------------

// Every global access of the kernels goes through a buffer resource that
// covers one tile: its base address is wave-uniform (scalar registers, one
// scalar add per tile), lanes add a 32-bit byte offset that stays the same
// from tile to tile, and an access past the tile's bytes reads 0 and writes
// nothing.  POL is the cache-policy operand (see cache_policy()).
struct TileRef {
  __amdgpu_buffer_rsrc_t r;
};

// Dword 3 of a buffer resource on gfx9 parts: 32-bit data format, the rest 0.
constexpr int kBufferResourceDword3 = 0x00020000;

__device__ __forceinline__ TileRef tile_ref(const void* base, uint32_t bytes) {
  return {__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferResourceDword3)};
}

// Cache-policy operand of the memory instructions: 0 = default (cached,
// write-back), kNT = non-temporal (streamed through once).  Other values are
// the raw operand (bit 0 and bit 4 set the coherence scope of a store).
constexpr int kNT = 2;
template <int POL>
constexpr int cache_policy() {
  return POL;
}

template <int NT>
__device__ __forceinline__ u32x4 ld16(TileRef t, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ u32x2 ld8(TileRef t, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ uint32_t ld4(TileRef t, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ uint32_t ld2(TileRef t, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ void st16(TileRef t, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ void st8(TileRef t, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ void st4(TileRef t, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ void st2(TileRef t, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, t.r, (int)off, 0, cache_policy<NT>());
}
template <int NT>
__device__ __forceinline__ void st1(TileRef t, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)v, t.r, (int)off, 0, cache_policy<NT>());
}

// ---------------------------------------------------------------------------
// 8-bit codes (INT8, ASYM8): a lane's block is 32 contiguous bytes, so loading
// or storing it directly would make every 16-byte access of the wave stride by
// 32 bytes.  Instead the wave moves row-order 16-byte chunks (lane l: chunks
// l and 64 + l, coalesced) and exchanges them through a wave-private 2 KB LDS
// region (lane l: chunks 2l and 2l + 1), padded like the tile: chunk c sits in
// slot c + c / 16, so lane l's row-order slots are l + l / 16 (+ 68) and its
// block-order slots 2l + l / 8 (+ 1), distinct modulo 16 within every 16 lanes.
// ---------------------------------------------------------------------------

template <int F>
constexpr bool kStaged = Format<F>::kCodeBits == 8;

constexpr int kStageSlots = kChunks / 2 + kChunks / 32;

// Row-order chunks (held in blk.w[0..3] = chunk l, blk.w[4..7] = chunk 64 + l)
// to the lane's own block (its 32 code bytes in order).  tl: 128 chunks.
__device__ __forceinline__ void stage_codes_in(u32x4* tl, uint32_t lane, CodeBlock<8>& blk) {
  const uint32_t rs = lane + (lane >> 4), bs = 2 * lane + (lane >> 3);
  tl[rs] = u32x4{blk.w[0], blk.w[1], blk.w[2], blk.w[3]};
  tl[rs + 68] = u32x4{blk.w[4], blk.w[5], blk.w[6], blk.w[7]};
  wave_lds_sync();
  const u32x4 a = tl[bs], b = tl[bs + 1];
  wave_lds_sync();
  blk.w[0] = a.x; blk.w[1] = a.y; blk.w[2] = a.z; blk.w[3] = a.w;
  blk.w[4] = b.x; blk.w[5] = b.y; blk.w[6] = b.z; blk.w[7] = b.w;
}

// The lane's block to row-order chunks, stored coalesced at tile + 16 * lane
// and tile + 1024 + 16 * lane.
template <int NT>
__device__ __forceinline__ void stage_codes_out(u32x4* tl, uint32_t lane, const CodeBlock<8>& blk, TileRef tile) {
  const uint32_t rs = lane + (lane >> 4), bs = 2 * lane + (lane >> 3);
  tl[bs] = u32x4{blk.w[0], blk.w[1], blk.w[2], blk.w[3]};
  tl[bs + 1] = u32x4{blk.w[4], blk.w[5], blk.w[6], blk.w[7]};
  wave_lds_sync();
  const u32x4 a = tl[rs], b = tl[rs + 68];
  wave_lds_sync();
  st16<NT>(tile, 16 * lane, a);
  st16<NT>(tile, 1024 + 16 * lane, b);
}

// Codes of block g and its scale.  For the asymmetric formats `scale`
// receives one dword of the tile's 48-byte scale / zero-point region (dword
// min(g & 15, 11)), and group_meta() later hands every lane its group's
// values: one memory instruction instead of a 2-byte and a 1-byte load.
template <int F, int NT>
__device__ __forceinline__ void load_block(TileRef tile, uint32_t g, Block<F>& blk, uint32_t& scale) {
  constexpr int BITS = Format<F>::kCodeBits;
  if constexpr (BITS == 4) {
    const u32x4 v = ld16<NT>(tile, 16 * g);
    blk.w[0] = v.x; blk.w[1] = v.y; blk.w[2] = v.z; blk.w[3] = v.w;
  } else if constexpr (BITS == 8) {
    // row-order chunks g and 64 + g; stage_codes_in() turns them into block g
    const u32x4 a = ld16<NT>(tile, 16 * g);
    const u32x4 b = ld16<NT>(tile, 1024 + 16 * g);
    blk.w[0] = a.x; blk.w[1] = a.y; blk.w[2] = a.z; blk.w[3] = a.w;
    blk.w[4] = b.x; blk.w[5] = b.y; blk.w[6] = b.z; blk.w[7] = b.w;
  } else {
    const u32x2 lw = ld8<NT>(tile, 8 * g);
    blk.low[0] = lw.x; blk.low[1] = lw.y;
    blk.high = ld4<NT>(tile, Format<3>::kHighOffset + 4 * g);
  }
  if constexpr (Format<F>::kAsym) {
    static_assert(Format<F>::kZeroOffset == Format<F>::kScaleOffset + 32, "scales then zero points");
    const uint32_t j = (g & 15) < 11 ? (g & 15) : 11;
    scale = ld4<NT>(tile, Format<F>::kScaleOffset + 4 * j);
  } else {
    scale = ld2<NT>(tile, Format<F>::kScaleOffset + 2 * g);
  }
}

// An INT3 tile held as 16 bytes per lane (bytes 16g .. 16g + 15 in lane g;
// lanes 56..63, past the tile, hold zeros) to lane g's block and scale,
// through the wave's LDS.
__device__ __forceinline__ void stage_int3_in(u32x4* tl, uint32_t g, u32x4 raw, CodeBlock<3>& blk, uint32_t& scale) {
  tl[g] = raw;
  wave_lds_sync();
  const uint32_t* w = reinterpret_cast<const uint32_t*>(tl);
  const uint32_t l0 = w[2 * g], l1 = w[2 * g + 1], h = w[Format<3>::kHighOffset / 4 + g];
  const uint32_t s = reinterpret_cast<const uint16_t*>(tl)[Format<3>::kScaleOffset / 2 + g];
  wave_lds_sync();
  blk.low[0] = l0;
  blk.low[1] = l1;
  blk.high = h;
  scale = s;
}

// What the decode of lane g's block needs from its group's scale s and zero
// point z: s for even values and s * 2^-kOddShift for odd ones (fp32), and the
// fp16 pairs -(1024 + z) and -(1024 + 16 z) (the pattern 0xE400 | c is
// -(1024 + c) for c < 1024).
struct AsymMeta {
  float d, dodd;
  f16x2 nz, nzo;
};

// Byte selectors (v_perm_b32) that pick lane g's group out of the two dwords
// group_meta() fetches: the scale's two bytes, and z under 0xE4 bytes twice.
struct MetaSel {
  uint32_t scale, zero;
};
__device__ __forceinline__ MetaSel meta_sel(uint32_t g) {
  const uint32_t grp = g >> 2, sb = 2 * (grp & 1), zb = grp & 3;
  return {sb | ((sb + 1) << 8) | 0x0C0C0000u, zb | (4u << 8) | (zb << 16) | (4u << 24)};
}

// The group metadata of lane g's block, from the dwords load_block() left in
// the lanes: dwords 0..7 hold the 16 fp16 scales (two each), dwords 8..11 the
// 16 zero points (four each).  Every lane of the wave takes part (cross-lane
// permutes).
template <int F>
__device__ __forceinline__ AsymMeta group_meta(uint32_t m, uint32_t g, const MetaSel& sel) {
  const uint32_t grp = g >> 2;
  const uint32_t sdw = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((grp >> 1) << 2), (int)m);
  const uint32_t zdw = (uint32_t)__builtin_amdgcn_ds_bpermute((int)((8 + (grp >> 2)) << 2), (int)m);
  constexpr uint32_t kE4 = 0xE4E4E4E4u;
  AsymMeta a;
  a.d = (float)__builtin_bit_cast(_Float16, (uint16_t)__builtin_amdgcn_perm(sdw, sdw, sel.scale));
  a.dodd = a.d * (1.0f / (1 << Format<F>::kOddShift));
  a.nz = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kE4, zdw, sel.zero));
  // 4-bit zero points: z << 4 stays within its byte
  a.nzo = Format<F>::kOddShift ? __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(kE4, zdw << 4, sel.zero)) : a.nz;
  return a;
}

// Stores block g; for the asymmetric formats the first lane of each group
// stores the group's scale and zero point (scale bits | zero point << 16).
// 8-bit codes are stored by stage_codes_out(), only their scale here.
template <int F, int NT>
__device__ __forceinline__ void store_block(TileRef tile, uint32_t g, const Block<F>& blk, uint32_t scale) {
  constexpr int BITS = Format<F>::kCodeBits;
  if constexpr (BITS == 4) {
    st16<NT>(tile, 16 * g, u32x4{blk.w[0], blk.w[1], blk.w[2], blk.w[3]});
  } else if constexpr (BITS == 8) {
    // the codes go through stage_codes_out(); only the scale is stored here
  } else {
    st8<NT>(tile, 8 * g, u32x2{blk.low[0], blk.low[1]});
    st4<NT>(tile, Format<3>::kHighOffset + 4 * g, blk.high);
  }
  if constexpr (Format<F>::kAsym) {
    if ((g & 3) == 0) {
      const uint32_t grp = g >> 2;
      st2<NT>(tile, Format<F>::kScaleOffset + 2 * grp, scale);
      st1<NT>(tile, Format<F>::kZeroOffset + grp, scale >> 16);
    }
  } else {
    st2<NT>(tile, Format<F>::kScaleOffset + 2 * g, scale);
  }
}

// fp32 of an fp16 scale held in the low 16 bits.
__device__ __forceinline__ float scale_f32(uint32_t s) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)s);
}

}  // namespace qr
