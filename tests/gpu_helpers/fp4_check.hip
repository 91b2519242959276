// Test helper (not part of the library): checks the library's FP4 device
// functions against definitions written here.
//   - fp4_pack (gfx950 v_cvt_scalef32_pk_fp4_f32 with scale 1.0) on every
//     fp32 bit pattern that is not a NaN: the E2M1 value nearest to the input
//     (ties to an even mantissa), magnitudes above 6 saturating to 6, the sign
//     bit kept; low nibble from the first operand, the byte at the selected
//     position, the other bytes of the destination unchanged.
//   - fp4_unpack on every byte at every position: the E2M1 values of the two
//     nibbles, signs included.
//   - fp4_block_scale for every positive finite fp16 and bf16 block maximum:
//     scale bits equal to fp16(min(m / 6, 65504)) with a correctly rounded
//     division, and the multiplier equal to 1.0f / d.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qr_codec.hpp"

// E2M1 code by comparing |v| with the midpoints between neighbouring
// magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; a midpoint goes to the neighbour with
// the even mantissa (0, 1, 2 and 4 have mantissa 0).
__device__ uint32_t ref_code(float v) {
  const float a = __builtin_fabsf(v);
  uint32_t m;
  if (a <= 0.25f) m = 0;
  else if (a < 0.75f) m = 1;
  else if (a <= 1.25f) m = 2;
  else if (a < 1.75f) m = 3;
  else if (a <= 2.5f) m = 4;
  else if (a < 3.5f) m = 5;
  else if (a <= 5.0f) m = 6;
  else m = 7;
  return ((__builtin_bit_cast(uint32_t, v) >> 31) << 3) | m;
}

__device__ float ref_value(uint32_t c) {
  const float mag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  const float a = mag[c & 7];
  return (c & 8) ? -a : a;
}

__device__ __forceinline__ uint32_t pack_sel(int sel, uint32_t old, float a, float b) {
  switch (sel) {
    case 0: return qr::fp4_pack<0>(old, a, b);
    case 1: return qr::fp4_pack<1>(old, a, b);
    case 2: return qr::fp4_pack<2>(old, a, b);
    default: return qr::fp4_pack<3>(old, a, b);
  }
}

// counters[0]: mismatches; counters[1]: smallest mismatching pattern
__global__ void fp4_pack_check(uint32_t* counters) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < (1ull << 32); p += stride) {
    const uint32_t bits = (uint32_t)p;
    if ((bits & 0x7F800000u) == 0x7F800000u && (bits & 0x007FFFFFu)) continue;  // NaN
    const float a = __builtin_bit_cast(float, bits);
    const float b = -a;
    const int sel = (int)(bits & 3);
    const uint32_t old = 0xA55AC33Cu;
    const uint32_t got = pack_sel(sel, old, a, b);
    const uint32_t byte = ref_code(a) | (ref_code(b) << 4);
    const uint32_t want = (old & ~(0xFFu << (8 * sel))) | (byte << (8 * sel));
    if (got != want) {
      atomicAdd(&counters[0], 1u);
      atomicMin(&counters[1], bits);
    }
  }
}

// counters[2]: mismatches over 256 bytes x 4 positions
__global__ void fp4_unpack_check(uint32_t* counters) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;  // 0 .. 1023
  if (t >= 1024) return;
  const uint32_t byte = t & 255, sel = t >> 8;
  const uint32_t w = (0x5A5A5A5Au & ~(0xFFu << (8 * sel))) | (byte << (8 * sel));
  qr::f32x2 v;
  switch (sel) {
    case 0: v = qr::fp4_unpack<0>(w); break;
    case 1: v = qr::fp4_unpack<1>(w); break;
    case 2: v = qr::fp4_unpack<2>(w); break;
    default: v = qr::fp4_unpack<3>(w); break;
  }
  const float lo = ref_value(byte & 15), hi = ref_value(byte >> 4);
  // copies first: this clang lowers __builtin_bit_cast of a vector element
  // expression (v.y) as element 0
  const float vx = v.x, vy = v.y;
  if (__builtin_bit_cast(uint32_t, vx) != __builtin_bit_cast(uint32_t, lo) ||
      __builtin_bit_cast(uint32_t, vy) != __builtin_bit_cast(uint32_t, hi))
    atomicAdd(&counters[2], 1u);
}

// counters[3]: fp16 maxima with a wrong scale or multiplier; counters[4]: bf16 maxima
__global__ void fp4_scale_check(uint32_t* counters) {
  const uint32_t h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h == 0 || h >= 0x7F80) return;
  for (int dt = 0; dt < 2; ++dt) {
    if (dt == 0 && h >= 0x7C00) continue;
    const float m = dt == 0 ? (float)__builtin_bit_cast(_Float16, (uint16_t)h) : __builtin_bit_cast(float, h << 16);
    float t = m / 6.0f;
    if (t > 65504.0f) t = 65504.0f;
    const _Float16 want = (_Float16)t;
    float d, e;
    const uint32_t got = qr::fp4_block_scale(m, d, e);
    const float dw = (float)want;
    const float ew = dw == 0.0f ? 0.0f : 1.0f / dw;
    if (got != (uint32_t)__builtin_bit_cast(uint16_t, want) || d != dw || e != ew) atomicAdd(&counters[3 + dt], 1u);
  }
}

// counters: 5 uint32 in device memory, zero except counters[1] = 0xFFFFFFFF.
extern "C" int qr_test_fp4_check(uint32_t* counters) {
  hipLaunchKernelGGL(fp4_pack_check, dim3(16384), dim3(256), 0, 0, counters);
  hipLaunchKernelGGL(fp4_unpack_check, dim3(4), dim3(256), 0, 0, counters);
  hipLaunchKernelGGL(fp4_scale_check, dim3(0x7F80 / 256 + 1), dim3(256), 0, 0, counters);
  return (int)hipDeviceSynchronize();
}
