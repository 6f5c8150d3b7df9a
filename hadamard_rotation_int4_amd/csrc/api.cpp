// Host-only part of the C ABI: version, status strings, width factorisation.
#include <math.h>

#include "common.hpp"

namespace qr {

float norm_constant(int32_t d) { return (float)(1.0 / sqrt((double)d)); }

}  // namespace qr

extern "C" int qr_abi_version(void) { return QR_ABI_VERSION; }

extern "C" const char* qr_status_str(int status) {
  switch (status) {
    case QR_OK: return "QR_OK";
    case QR_ERR_NULL: return "QR_ERR_NULL: a required pointer is NULL";
    case QR_ERR_SHAPE: return "QR_ERR_SHAPE: invalid or inconsistent sizes";
    case QR_ERR_UNSUPPORTED: return "QR_ERR_UNSUPPORTED: size not implemented by the kernels";
    case QR_ERR_ALIGN: return "QR_ERR_ALIGN: pointer or stride misaligned";
    case QR_ERR_LAUNCH: return "QR_ERR_LAUNCH: kernel launch failed";
    case QR_ERR_ARG: return "QR_ERR_ARG: scalar argument out of range";
    case QR_ERR_SCRATCH: return "QR_ERR_SCRATCH: needs more than the library's static scratch";
    default: return "unknown qr_status";
  }
}

extern "C" qr_status qr_hadamard_factor(int32_t d, int32_t* log2_pow2, int32_t* m) {
  if (!log2_pow2 || !m) return QR_ERR_NULL;
  int n = 0, mm = 0;
  if (!qr::factor_width(d, &n, &mm)) return QR_ERR_UNSUPPORTED;
  *log2_pow2 = n;
  *m = mm;
  return QR_OK;
}
