// Host-only helpers of the C-ABI: version and status text.
#include "common.h"

extern "C" const char* uep_version(void) { return "uep 0.1.0 (gfx950)"; }

extern "C" const char* uep_status_string(uep_status s) {
  switch (s) {
    case UEP_OK: return "ok";
    case UEP_EINVAL: return "invalid argument";
    case UEP_EGEOM: return "unsupported geometry";
    case UEP_EWORKSPACE: return "workspace too small";
    case UEP_EHIP: return "HIP launch or runtime failure";
    default: return "unknown status";
  }
}
