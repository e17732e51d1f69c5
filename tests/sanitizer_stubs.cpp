// Test-only stand-ins for the kernel dispatchers, for the host-code sanitizer build of the C ABI
// (tests/test_sanitizers.py): that build has no device code, and its calls are all rejected before
// any launch, so these are never reached; each reports an error if one were.
#include "kia_launch.hpp"

namespace kia {
#define KIA_STUB(C)                                                                                   \
  template <> hipError_t forward_cal<C>(const Problem&, const FwdArgs&, hipStream_t) { return hipErrorNotSupported; } \
  template <> hipError_t bins_cal<C>(const Problem&, const BinsArgs&, hipStream_t) { return hipErrorNotSupported; }   \
  template <> hipError_t dq_cal<C>(const Problem&, const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
KIA_STUB(MINMAX)
KIA_STUB(FWM)
KIA_STUB(FWM_FLOOR)
KIA_STUB(FWM_RES)
KIA_STUB(EXPB)
hipError_t launch_dkdv(const Problem&, const BwdArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_flash_forward(const Problem&, const FlashArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_flash_backward(const Problem&, const FlashArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace kia
