// Library-wide entry points: status strings, ABI version, device queries.
#include <atomic>

#include "common.hpp"

namespace specv {

// Compute units of the current device, cached per device (relaxed atomics:
// concurrent first calls store the same value).
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace specv

extern "C" const char* spec_status_string(spec_status_t s) {
  switch (s) {
    case SPEC_OK: return "ok";
    case SPEC_E_NULL: return "a required pointer is NULL";
    case SPEC_E_SHAPE: return "a size argument is out of range";
    case SPEC_E_DTYPE: return "unsupported dtype / head_dim combination";
    case SPEC_E_VALUE: return "bad scalar argument (temperature or scale)";
    case SPEC_E_WORKSPACE: return "workspace NULL or smaller than required";
    case SPEC_E_HIP: return "a HIP runtime call or kernel launch failed";
    case SPEC_E_UNSUPPORTED: return "configuration not supported on the current device";
    case SPEC_E_SCRATCH:
      return "the call needs more device scratch than the library's fixed array holds";
    default: return "unknown status";
  }
}

extern "C" int32_t spec_abi_version(void) { return SPEC_ABI_VERSION; }
