// Library-wide entry points: ABI version and status strings.
#include "common.hpp"

extern "C" int32_t csa2_abi_version(void) { return 1; }

extern "C" const char* csa2_status_str(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument (null pointer, non-positive size or bad value)";
    case CSA2_ESHAPE: return "unsupported shape";
    case CSA2_EALIGN: return "pointer or stride not aligned as required";
    case CSA2_EWORKSPACE: return "workspace missing or too small";
    case CSA2_ELAUNCH: return "kernel launch failed";
    case CSA2_ESCRATCH: return "shape needs more than the fixed scratch array of the allocation-free call";
    default: return "unknown status";
  }
}
