// kda_prefill_mfma_gate.hip -- launches of the chunked KDA prefill with the
// gate given as its logit (fp32 or bf16), g = g_min sigmoid(x) formed in the
// kernel, with or without the q/k normalisation.  A separate translation unit, so that these variants can take the
// layout and the scheduling strategy that suit their heavier k-side (one
// exponential and one reciprocal more per value): two k-side waves per SIMD,
// each on one 16-channel tile, and the default strategy.
#define KDA_KSIDE_WAVES_PER_SIMD 2
#include "kda_prefill_mfma.h"

namespace kda {

hipError_t launch_prefill_mfma_gate(const PrefillArgs &a, dim3 grid, hipStream_t s) {
    if (a.gate == kGateLogitF32 && a.qk_norm)
        hipLaunchKernelGGL((prefill_mfma_qknorm_kernel<kGateLogitF32>), grid, dim3(kThreads), 0, s, a);
    else if (a.gate == kGateLogitF32)
        hipLaunchKernelGGL((prefill_mfma_kernel<false, kGateLogitF32, kFull>), grid, dim3(kThreads), 0, s, a);
    else if (a.gate == kGateLogitBf16 && a.qk_norm)
        hipLaunchKernelGGL((prefill_mfma_qknorm_kernel<kGateLogitBf16>), grid, dim3(kThreads), 0, s, a);
    else if (a.gate == kGateLogitBf16)
        hipLaunchKernelGGL((prefill_mfma_kernel<false, kGateLogitBf16, kFull>), grid, dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
