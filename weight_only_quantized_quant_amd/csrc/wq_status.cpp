// Status strings of the C ABI.
#include "wq.h"

extern "C" const char* wq_status_string(int status) {
  switch (status) {
    case WQ_OK: return "WQ_OK";
    case WQ_EINVAL: return "WQ_EINVAL: invalid shape, size, pointer or divisibility";
    case WQ_EALIGN: return "WQ_EALIGN: base pointer not 16-byte aligned";
    case WQ_EUNSUPPORTED: return "WQ_EUNSUPPORTED: dtype/block/group combination not supported";
    case WQ_EHIP: return "WQ_EHIP: HIP launch or runtime error";
    default: return "unknown wq_status";
  }
}
