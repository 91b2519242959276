// qr_fp4.hip -- instantiations for the FP4 E2M1 block codec (format 36:
// 32-value blocks with an fp16 scale, E2M1 codes packed as INT4 nibbles, the
// gfx950 scaled FP4 conversions; "QuickReduce INT3 quantization and
// benchmarking on MI355", introduction: a hardware FP4 path on MI355 that is
// interchangeable with INT4).
#include "qr_kernels.hpp"

namespace qr {

qr_status launch_encode_fp4(int dt, const void* x, void* p, size_t ntiles, hipStream_t st) {
  return launch_encode<36>(dt, x, p, ntiles, st);
}

qr_status launch_decode_fp4(int dt, const void* p, void* y, size_t ntiles, hipStream_t st) {
  return launch_decode<36>(dt, p, y, ntiles, st);
}

qr_status launch_reduce_fp4(int dt, const ReduceArgs& a, hipStream_t st) {
  return launch_reduce<36, 36>(dt, a, st);
}

}  // namespace qr
