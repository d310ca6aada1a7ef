// prefill_bf16.hip -- bf16 MFMA chunked prefill (gfx950).  Placeholder until
// the kernel lands: not selected by the dispatcher.
#include "gdn_internal.h"

namespace gdn {

const bool kHaveBf16Mfma = false;

Bf16Plan plan_prefill_bf16(int64_t, int32_t, int32_t, int32_t, bool) {
  return Bf16Plan{1, 0};
}

hipError_t launch_prefill_bf16(const PrefillParams&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace gdn
