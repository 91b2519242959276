// Test helper (not part of the library): runs the library's own block-scale
// device function over every positive finite fp16 scale and counts where the
// encode multiplier differs from the correctly rounded IEEE quotient 1.0f / d,
// or the scale bits differ from d.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qr_codec.hpp"

template <int BITS>
__global__ void scale_check(uint32_t* bad_e, uint32_t* bad_d) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x + 1;  // fp16 bits 0x0001 .. 0x7BFF
  if (h > 0x7BFF) return;
  const float dv = (float)__builtin_bit_cast(_Float16, (uint16_t)h);
  float d, e;
  const uint32_t bits = qr::block_scale<BITS>(dv * (float)qr::Format<BITS>::kQ, d, e);
  if (e != 1.0f / dv) atomicAdd(bad_e, 1u);
  if (bits != (uint32_t)h || d != dv) atomicAdd(bad_d, 1u);
}

// counters: 6 uint32 (bad_e, bad_d) for INT3, INT4, INT8; device memory.
extern "C" int qr_test_scale_check(uint32_t* counters) {
  const dim3 grid(0x7BFF / 256 + 1), block(256);
  hipLaunchKernelGGL(scale_check<3>, grid, block, 0, 0, counters + 0, counters + 1);
  hipLaunchKernelGGL(scale_check<4>, grid, block, 0, 0, counters + 2, counters + 3);
  hipLaunchKernelGGL(scale_check<8>, grid, block, 0, 0, counters + 4, counters + 5);
  return (int)hipDeviceSynchronize();
}
