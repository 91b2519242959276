// qr_asym.hip -- instantiations for the asymmetric group codec (formats 20 =
// 4-bit codes, 24 = 8-bit codes; 128-value groups with a scale and a zero
// point, the "Flash Communication" review of arXiv 2412.04964, fields
// pith_summary / key_machinery).  Compiled once per input format
// (QR_ASYM_IN = 20, 24) so that the instantiations build in parallel; the
// first object also holds encode and decode.
#include "qr_kernels.hpp"

#ifndef QR_ASYM_IN
#error "QR_ASYM_IN (asymmetric input format, 20 or 24) must be defined"
#endif

namespace qr {

#define QR_CAT2(a, b) a##b
#define QR_CAT(a, b) QR_CAT2(a, b)

qr_status QR_CAT(launch_reduce_asym_from, QR_ASYM_IN)(int fmt_out, int dt, const ReduceArgs& a,
                                                      hipStream_t st) {
  constexpr int BI = QR_ASYM_IN;
  switch (fmt_out) {
    case QR_ASYM4: return launch_reduce<BI, 20>(dt, a, st);
    case QR_ASYM8: return launch_reduce<BI, 24>(dt, a, st);
    default: return QR_ERR_UNSUPPORTED;
  }
}

#if QR_ASYM_IN == 20
qr_status launch_encode_asym(int fmt, int dt, const void* x, void* p, size_t ntiles, hipStream_t st) {
  return fmt == QR_ASYM4 ? launch_encode<20>(dt, x, p, ntiles, st) : launch_encode<24>(dt, x, p, ntiles, st);
}

qr_status launch_decode_asym(int fmt, int dt, const void* p, void* y, size_t ntiles, hipStream_t st) {
  return fmt == QR_ASYM4 ? launch_decode<20>(dt, p, y, ntiles, st) : launch_decode<24>(dt, p, y, ntiles, st);
}
#endif

}  // namespace qr
