// Host-only stand-ins for a CPU AddressSanitizer build of api.cpp: the
// kernel launchers, the validation hooks and the HIP runtime calls api.cpp
// makes.  Every launcher and runtime call reports a failure, so a call that
// passes the host-side checks returns SPECV_E_HIP; no device is ever touched.
#include "specverify.h"
#include "sv_internal.h"

namespace sv {
hipError_t launch_sweep_lse(const Params&, int, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorInvalidValue; }
hipError_t launch_sweep_argmax(const Params&, int, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorInvalidValue; }
hipError_t launch_verify(const Params&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_exact(const Params&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_short(const Params&, int, hipStream_t, hipEvent_t, hipEvent_t) { return hipErrorInvalidValue; }
hipError_t launch_greedy_scan(const Params&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_round_accept(const Params&, int, bool, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_position_stats(const Params&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_tree_scan(const Params&, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_tree_round(const Params&, int, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_sweep_argmax_tree(const Params&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_ngram(const int32_t*, const int32_t*, int, int, int, int, int, int, int32_t*, int32_t*,
                        hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_ngram_map(void*, int, const int32_t*, const int32_t*, const int32_t*, int, int, int, int, int,
                            int, int32_t*, int32_t*, int32_t*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_tree_mask(const int32_t*, int, int, uint8_t*, int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_validate(const Params&, int, bool, unsigned long long*, hipStream_t) { return hipErrorInvalidValue; }
bool debug_enabled_flag(int* set_to) {
  static int on = 0;
  const bool prev = on != 0;
  if (set_to) on = *set_to ? 1 : 0;
  return prev;
}
unsigned long long* debug_counters_ptr() {  // a device array's address (none here)
  static unsigned long long counters[SPECV_DEBUG_COUNTERS];
  return counters;
}
}  // namespace sv

extern "C" {
hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
hipError_t hipGetSymbolAddress(void** ptr, const void*) {
  *ptr = nullptr;
  return hipErrorInvalidSymbol;
}
hipError_t hipDeviceSynchronize(void) { return hipErrorInvalidValue; }
hipError_t hipMemcpy(void*, const void*, size_t, hipMemcpyKind) { return hipErrorInvalidValue; }
}
