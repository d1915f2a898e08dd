// Host-only stand-ins for the device half of libfm (the functions that
// fm_launch.hip defines), so that the plan builder and the C ABI can be
// built with g++ under AddressSanitizer / UndefinedBehaviorSanitizer.
// Test infrastructure: never linked into the library.
#include "fm_internal.h"

namespace fm {

int upload_plan(Plan&) { return set_error(FM_E_NODEVICE, "host-only build"); }

void free_plan_device(Plan& p) {
  p.d_block = nullptr;
  p.has_device = false;
}

int launch_forward(const Plan& p, const void*, int, int64_t, int64_t, void*, void*) {
  if (!p.has_device) return set_error(FM_E_NODEVICE, "plan was built without device tables");
  return set_error(FM_E_HIP, "host-only build");
}

int launch_backward(const Plan& p, const float*, int64_t, int64_t, const float*, float*, void*) {
  if (!p.has_device) return set_error(FM_E_NODEVICE, "plan was built without device tables");
  return set_error(FM_E_HIP, "host-only build");
}

}  // namespace fm
