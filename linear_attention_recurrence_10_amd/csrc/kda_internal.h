// kda_internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int kChunk = 16;  // tokens per chunk: g_min = -5 keeps exp(+-16*5) inside bf16 range

// How the per-channel forget gate is given: the fp32 log-decay g itself, or
// its logit x (fp32 or bf16) with g = g_min * sigmoid(x) formed in the kernel.
enum GateMode { kGateLogDecay = 0, kGateLogitF32 = 1, kGateLogitBf16 = 2 };

struct PrefillArgs {
    const void *q, *k, *v;   // [B,T,H,D] in dtype
    const void *g;           // [B,T,H,D]: fp32 log-decay, or logits (gate)
    int gate;                // GateMode
    float g_min;             // floor of the gate for the logit modes
    const float *beta;       // [B,T,H]
    const float *h0;         // [B,H,D,D] or null
    float *o;                // [B,T,H,D]
    float *hT;               // [B,H,D,D] or null (may equal h0)
    float *ckpt;             // [n_ckpt,B,H,D,D] or null: state after every ckpt_every chunks
    int64_t ckpt_every;      // chunks between checkpoints (>= 1 when ckpt is set)
    int64_t n_ckpt;          // checkpoints to write
    int64_t B, T, H;
    int D;
    bool bf16;
    float scale;
    uint32_t epoch;          // launch tag of the value slices' pacing (set by the MFMA launcher)
    bool qk_norm;            // q and k are used as x / max(||x||, eps) (per token and head)
    float qk_eps2;           // eps^2 of that normalisation
};

struct DecodeArgs {
    const void *q, *k, *v;   // [B,H,D]
    const float *g;          // [B,H,D]
    const float *beta;       // [B,H]
    float *state;            // [B,H,D,D], in place
    float *o;                // [B,H,D]
    int64_t B, H;
    int D;
    bool bf16;
    float scale;
    bool qk_norm;            // q and k are used as x / max(||x||, eps)
    float qk_eps2;           // eps^2 of that normalisation
};

// The backward pass (kda_bwd.hip): gradients of every input given dO and dhT.
struct BwdArgs {
    const void *q, *k, *v;   // [B,T,H,D] in dtype
    const float *g, *beta;   // [B,T,H,D], [B,T,H]
    const float *h0;         // [B,H,D,D] or null
    const float *dO;         // [B,T,H,D]
    const float *dhT;        // [B,H,D,D] or null (zero)
    const float *ckpt;       // [T / 16, B,H,D,D]: the state after every 16 tokens
    float *dq, *dk, *dv, *dg, *dbeta;  // like q, k, v, g, beta
    float *dh0;              // [B,H,D,D] or null
    float *part;             // per-slice sums over columns: [slices][3 planes of B T H D, then B T H]
    int64_t part_stride;     // floats per slice
    int64_t part_plane;      // B T H D
    int64_t B, T, H;
    int D;
    bool bf16;
    float scale;
};

// Each launcher returns hipSuccess or the launch error; all are asynchronous.
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);
hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s);
hipError_t launch_prefill_mfma_gate(const PrefillArgs &a, dim3 grid, hipStream_t s);  // gate-logit variants
bool prefill_mfma_supported(const PrefillArgs &a);
// fp32 inputs at d = 128 on the fp32 matrix cores (kda_prefill_f32.hip)
hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s);
bool prefill_f32_supported(const PrefillArgs &a);
// KDA_DISABLE_MFMA=1 in the environment (read once per process) routes every
// prefill to the fp32 vector-ALU kernel: a comparison knob for tests
bool prefill_mfma_disabled();
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
// Segmented prefill helpers (kda_kcp.hip).
// The fixed per-device workspace of kda_chunk_fwd_kcp_noalloc: 32 MiB, room
// for three state sets of B * n_seg * H <= 170 heads at d = 128.
constexpr uint64_t kKcpScratchBytes = 32ull << 20;
constexpr int kMaxDevices = 64;
// Its device address on the current device (looked up once per device).
hipError_t kcp_scratch(void **ptr);
hipError_t launch_fill_identity(float *states, int64_t n, int D, hipStream_t s);
hipError_t launch_kcp_combine(const float *M, const float *Bs, const float *h0, float *S_in, float *hT, int64_t B,
                              int64_t P, int64_t H, int D, hipStream_t s);

// g = g_min * sigmoid(x) = g_min / (1 + e^-x): the bounded scaled-sigmoid
// gate of the Kimi K3 paper digest (devpress.csdn.net), section 2.1 (1), with
// the hardware exp2 and reciprocal (about 1 ulp each).  x -> -inf gives 0,
// x -> +inf gives g_min.
__device__ __forceinline__ float gate_of_logit(float x, float g_min) {
    return g_min * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(x * -1.4426950408889634f));
}

// The factor of the q/k normalisation x / max(||x||, eps) from the sum of
// squares s = ||x||^2: 1 / max(||x||, eps) = rsqrt(max(s, eps^2)), with the
// hardware reciprocal square root (about 1 ulp).  eps^2 is a normal fp32
// number (the entry points keep eps in [1e-18, 1e18]), so the factor is finite.
__device__ __forceinline__ float norm_factor(float sumsq, float eps2) {
    return __builtin_amdgcn_rsqf(fmaxf(sumsq, eps2));
}

// bf16 (stored as raw 16-bit patterns) and fp32 element loads.
__device__ __forceinline__ float ld_elem(const uint16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float ld_elem(const float *p, int64_t i) { return p[i]; }

}  // namespace kda
