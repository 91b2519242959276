// Test helper (not part of the library): evaluates the library's asymmetric
// group parameters (scale bits, multiplier, zero point) for host-given
// (lo, hi) pairs, for comparison with the oracle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qr_codec.hpp"

template <int F>
__global__ void group_params_kernel(const float* lo, const float* hi, uint32_t* d_bits, float* e, uint32_t* z,
                                    int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float d, ee, zz;
  const uint32_t p = qr::group_params<F>(lo[i], hi[i], d, ee, zz);
  d_bits[i] = p & 0xffffu;
  e[i] = ee;
  z[i] = p >> 16;
}

// fmt: 20 (4-bit codes) or 24 (8-bit codes); all pointers device memory, n entries each.
extern "C" int qr_test_group_params(int fmt, const float* lo, const float* hi, uint32_t* d_bits, float* e,
                                    uint32_t* z, int n) {
  const dim3 grid((n + 255) / 256), block(256);
  if (fmt == 20)
    hipLaunchKernelGGL(group_params_kernel<20>, grid, block, 0, 0, lo, hi, d_bits, e, z, n);
  else if (fmt == 24)
    hipLaunchKernelGGL(group_params_kernel<24>, grid, block, 0, 0, lo, hi, d_bits, e, z, n);
  else
    return -1;
  return (int)hipDeviceSynchronize();
}
