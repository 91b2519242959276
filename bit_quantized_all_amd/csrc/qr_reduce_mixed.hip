// qr_reduce_mixed.hip -- instantiations of the fused reduction with the
// inputs in one format and the re-encoded sum in another (the "INT6"
// configuration of the Flash Communication review: INT4 reduce-scatter
// inputs, INT8 all-gather payload; every other pair of INT3/INT4/INT8 too).
// Compiled once per input format (QR_MIXED_IN = 3, 4, 8) so that the
// instantiations build in parallel.
#include "qr_kernels.hpp"

#ifndef QR_MIXED_IN
#error "QR_MIXED_IN (input format bits) must be defined"
#endif

namespace qr {

#define QR_CAT2(a, b) a##b
#define QR_CAT(a, b) QR_CAT2(a, b)

qr_status QR_CAT(launch_reduce_mixed_from, QR_MIXED_IN)(int fmt_out, int dt, const ReduceArgs& a,
                                                        hipStream_t st) {
  constexpr int BI = QR_MIXED_IN;
  switch (fmt_out) {
    case QR_INT3: if constexpr (BI != 3) return launch_reduce<BI, 3>(dt, a, st); break;
    case QR_INT4: if constexpr (BI != 4) return launch_reduce<BI, 4>(dt, a, st); break;
    case QR_INT8: if constexpr (BI != 8) return launch_reduce<BI, 8>(dt, a, st); break;
    default: break;
  }
  return QR_ERR_UNSUPPORTED;  // equal formats take the same-format path
}

}  // namespace qr
