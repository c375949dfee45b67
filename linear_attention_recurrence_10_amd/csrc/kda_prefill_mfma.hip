// kda_prefill_mfma.hip -- MFMA chunked prefill (not yet enabled).
#include "kda_internal.h"

namespace kda {

bool prefill_mfma_supported(const PrefillArgs &) { return false; }

hipError_t launch_prefill_mfma(const PrefillArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
