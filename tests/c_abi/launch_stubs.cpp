// launch_stubs.cpp -- stand-ins for the launch functions that the library's
// other translation units define, so that qr_api.hip links on its own for the
// host-sanitizer build of the argument checks.  A call that passes every
// check reaches one of them and returns QR_ERR_HIP, the sign that the call
// was accepted; no GPU work is launched.
#include <hip/hip_runtime.h>

#include "qr.h"
#include "qr_kernels.hpp"

namespace qr {
qr_status launch_reduce_mixed_from3(int, int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_reduce_mixed_from4(int, int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_reduce_mixed_from8(int, int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_encode_asym(int, int, const void*, void*, size_t, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_decode_asym(int, int, const void*, void*, size_t, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_reduce_asym_from20(int, int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_reduce_asym_from24(int, int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_encode_fp4(int, const void*, void*, size_t, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_decode_fp4(int, const void*, void*, size_t, hipStream_t) { return QR_ERR_HIP; }
qr_status launch_reduce_fp4(int, const ReduceArgs&, hipStream_t) { return QR_ERR_HIP; }
}  // namespace qr
