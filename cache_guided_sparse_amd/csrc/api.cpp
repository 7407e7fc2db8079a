// Host-side helpers of the C ABI (no device code).
#include <math.h>

#include "../../include/cgs.h"

extern "C" int cgs_ratio_to_count(double rho, int n) {
  if (n <= 0 || !(rho == rho)) return 0;
  const double k = ceil(rho * static_cast<double>(n) - 1e-9);
  if (k <= 0.0) return 0;
  if (k >= static_cast<double>(n)) return n;
  return static_cast<int>(k);
}

extern "C" const char* cgs_status_str(int status) {
  switch (status) {
    case CGS_OK: return "ok";
    case CGS_ERR_ARG: return "invalid argument";
    case CGS_ERR_SHAPE: return "size or count out of range";
    case CGS_ERR_WORKSPACE: return "workspace too small";
    case CGS_ERR_UNSUPPORTED: return "unsupported dtype, layout or size";
    case CGS_ERR_LAUNCH: return "kernel launch failed";
    case CGS_ERR_DATA: return "device data break a documented precondition";
    case CGS_ERR_TIMEOUT: return "a persistent kernel's bounded wait gave up";
    default: return "unknown status";
  }
}

extern "C" int cgs_version(void) { return 100; }
