// Library-wide C ABI entry points that launch nothing.
#include "dcu.h"

extern "C" const char* dcu_status_string(int status) {
  switch (status) {
    case DCU_OK: return "ok";
    case DCU_EINVAL: return "invalid argument";
    case DCU_EUNSUPPORTED: return "unsupported shape, dtype or alignment";
    case DCU_EWORKSPACE: return "workspace missing or too small";
    case DCU_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int dcu_version(void) { return 100; }  // 0.1.0
