// kda_prefill_mfma.hip -- launches of the chunked KDA prefill on the gfx950
// matrix cores (the kernel template is in kda_prefill_mfma.h): the fp32
// log-decay gate, with or without state checkpoints or the q/k
// normalisation, and the passes that write no o (those of the segmented
// prefill, and the checkpoint pass of the backward).
// The gate-logit variants live in kda_prefill_mfma_gate.hip.
#include <atomic>

#include "kda_prefill_mfma.h"

namespace kda {

// KDA_DISABLE_MFMA=1 in the environment routes every prefill to the fp32
// vector kernel (a comparison knob for tests); it is read once per process.
static const bool g_mfma_disabled = [] {
    const char *env = getenv("KDA_DISABLE_MFMA");
    return env && env[0] == '1';
}();

bool prefill_mfma_disabled() { return g_mfma_disabled; }

bool prefill_mfma_supported(const PrefillArgs &a) {
    // the kernel's 32-bit in-chunk byte offsets need kC * H * 128 * 4 < 2^31,
    // i.e. H < 65536 (the products are formed in 32 bits)
    if (a.D != kD || !a.bf16 || a.H >= 65536) return false;
    return !g_mfma_disabled;
}

hipError_t launch_prefill_mfma(const PrefillArgs &args, hipStream_t s) {
    static std::atomic<uint32_t> epochs{0};
    PrefillArgs a = args;
    a.epoch = epochs.fetch_add(1, std::memory_order_relaxed) + 1;
    if (a.epoch == 0) a.epoch = epochs.fetch_add(1, std::memory_order_relaxed) + 1;  // (0 means unpaced)
    const int64_t BH = a.B * a.H;
    const int64_t rounds = (BH + 7) / 8;
    const dim3 grid(static_cast<unsigned>(rounds * 8 * kNV));
    // checkpoints, and the passes without o, come with the fp32 log-decay gate
    // and without the q/k normalisation only (the entry points offer no other
    // combination); checkpoints always come with values
    const bool plain = a.gate == kGateLogDecay && !a.qk_norm;
    if ((!a.o || !a.v || a.ckpt) && !plain) return hipErrorInvalidValue;
    if (!a.v && (a.o || a.ckpt)) return hipErrorInvalidValue;
    if (a.ckpt && a.o)
        hipLaunchKernelGGL((prefill_mfma_kernel<true, kGateLogDecay, kFull>), grid, dim3(kThreads), 0, s, a);
    else if (a.ckpt)
        hipLaunchKernelGGL((prefill_mfma_kernel<true, kGateLogDecay, kNoOut>), grid, dim3(kThreads), 0, s, a);
    else if (a.gate != kGateLogDecay)
        return launch_prefill_mfma_gate(a, grid, s);
    else if (a.qk_norm)
        hipLaunchKernelGGL((prefill_mfma_qknorm_kernel<kGateLogDecay>), grid, dim3(kThreads), 0, s, a);
    else if (!a.v)
        hipLaunchKernelGGL((prefill_mfma_kernel<false, kGateLogDecay, kNoValue>), grid, dim3(kThreads), 0, s, a);
    else if (!a.o)
        hipLaunchKernelGGL((prefill_mfma_kernel<false, kGateLogDecay, kNoOut>), grid, dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((prefill_mfma_kernel<false, kGateLogDecay, kFull>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
