// prefill.hip -- chunked-prefill paged attention (bf16 MFMA).  Not built yet.
#include "pkv_internal.h"

namespace pkv {
hipError_t launch_prefill(const PrefillLaunch&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pkv
