// kda_api.cpp -- the C ABI declared in include/kda.h: argument validation,
// kernel selection and launch on the caller's stream.
#include "kda.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "kda_internal.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status fail(kda_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

kda_status ok() {
    g_last_error[0] = '\0';
    return KDA_OK;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    const char *name;
    const void *p;
    uint64_t bytes;
};

bool overlaps(const Span &a, const Span &b) {
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Product of positive sizes with an overflow check (false on overflow).
bool mul_ok(uint64_t &acc, int64_t x) {
    if (x < 0) return false;
    if (x != 0 && acc > UINT64_MAX / static_cast<uint64_t>(x)) return false;
    acc *= static_cast<uint64_t>(x);
    return true;
}

// Architecture check, cached per device ordinal: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[64];

kda_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return fail(KDA_ERR_DEVICE, "no current HIP device");
    if (dev < 64) {
        int st = g_arch[dev].load(std::memory_order_relaxed);
        if (st == 1) return KDA_OK;
        if (st == 2) return fail(KDA_ERR_DEVICE, "device %d is not gfx950", dev);
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return fail(KDA_ERR_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    const bool good = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) g_arch[dev].store(good ? 1 : 2, std::memory_order_relaxed);
    if (!good) return fail(KDA_ERR_DEVICE, "device %d is %s, this library is built for gfx950", dev, prop.gcnArchName);
    return KDA_OK;
}

// A tensor argument must be a device allocation that covers all of its bytes,
// so that a wrong pointer or size is rejected here instead of faulting the GPU.
kda_status check_device_span(const Span &s) {
    if (!s.p || s.bytes == 0) return KDA_OK;
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void *>(s.p)) != hipSuccess || base == nullptr) {
        (void)hipGetLastError();
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not a device allocation", s.name);
    }
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(base), p0 = reinterpret_cast<uintptr_t>(s.p);
    if (p0 + s.bytes > b0 + size)
        return fail(KDA_ERR_INVALID_ARGUMENT, "%s: %llu bytes from the pointer run past the end of its allocation",
                    s.name, static_cast<unsigned long long>(s.bytes));
    return KDA_OK;
}

kda_status check_spans(const Span *sp, int n) {
    for (int i = 0; i < n; ++i) {
        if (sp[i].p && !aligned16(sp[i].p))
            return fail(KDA_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", sp[i].name);
    }
    for (int i = 0; i < n; ++i) {
        kda_status st = check_device_span(sp[i]);
        if (st != KDA_OK) return st;
    }
    return KDA_OK;
}

kda_status launch_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(KDA_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

const char *kda_status_string(kda_status s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARGUMENT: return "KDA_ERR_INVALID_ARGUMENT";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_LAUNCH: return "KDA_ERR_LAUNCH";
        case KDA_ERR_DEVICE: return "KDA_ERR_DEVICE";
    }
    return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_last_error; }

int kda_version(void) { return 100; }  // 0.1.0

}  // extern "C"

namespace {

kda_status launch_prefill(const kda::PrefillArgs &a, hipStream_t s) {
    if (kda::prefill_mfma_supported(a)) return launch_status(kda::launch_prefill_mfma(a, s), "kda prefill (mfma)");
    if (kda::prefill_f32_supported(a) && !kda::prefill_mfma_disabled())
        return launch_status(kda::launch_prefill_f32(a, s), "kda prefill (fp32 mfma)");
    return launch_status(kda::launch_prefill_valu(a, s), "kda prefill (valu)");
}

// The prefill entry points: kda_chunk_fwd is this with no checkpoints.  With
// `out`, the validated arguments are returned instead of launched.  qk_eps > 0
// turns on the q/k normalisation with that floor (checked by the caller).
kda_status chunk_fwd(const void *q, const void *k, const void *v, const void *g, kda::GateMode gate, float g_min,
                     const float *beta, const float *h0, float *o, float *hT, float *ckpt, int64_t ckpt_every,
                     int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale,
                     void *stream, kda::PrefillArgs *out = nullptr, bool device_checks = true,
                     float qk_eps = 0.f, bool o_optional = false) {
    if (B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0 || T < 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "sizes must be positive (T >= 0): B=%lld T=%lld H=%lld Dk=%lld Dv=%lld",
                    (long long)B, (long long)T, (long long)H, (long long)Dk, (long long)Dv);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown in_dtype %d", static_cast<int>(in_dtype));
    if (Dk != Dv || (Dk != 16 && Dk != 128))
        return fail(KDA_ERR_UNSUPPORTED, "head dims Dk=%lld Dv=%lld: only Dk == Dv in {16, 128} is built",
                    (long long)Dk, (long long)Dv);
    if (T > 0 && (!q || !k || !v || !g || !beta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o must be non-null when T > 0");
    if (T > 0 && !o && !(o_optional && ckpt))
        return fail(KDA_ERR_INVALID_ARGUMENT, o_optional ? "o may be null only when ckpt is given"
                                                         : "q, k, v, g, beta and o must be non-null when T > 0");
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
    if (ckpt && (ckpt_every <= 0 || ckpt_every % kda::kChunk != 0))
        return fail(KDA_ERR_INVALID_ARGUMENT, "ckpt_every=%lld must be a positive multiple of %d",
                    (long long)ckpt_every, kda::kChunk);
    const int64_t n_ckpt = ckpt ? T / ckpt_every : 0;

    uint64_t n_tok = 1, n_state = 1;
    if (!mul_ok(n_tok, B) || !mul_ok(n_tok, T) || !mul_ok(n_tok, H) || !mul_ok(n_state, B) ||
        !mul_ok(n_state, H) || !mul_ok(n_state, Dk) || !mul_ok(n_state, Dv))
        return fail(KDA_ERR_INVALID_ARGUMENT, "tensor sizes overflow 64 bits");
    uint64_t n_qk = n_tok, n_v = n_tok;
    if (!mul_ok(n_qk, Dk) || !mul_ok(n_v, Dv) || n_qk > UINT64_MAX / 8)
        return fail(KDA_ERR_INVALID_ARGUMENT, "tensor sizes overflow 64 bits");
    if (B * H * 64 > INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "B*H too large for one launch");
    uint64_t n_ck = n_state;
    if (!mul_ok(n_ck, n_ckpt) || n_ck > UINT64_MAX / 4)
        return fail(KDA_ERR_INVALID_ARGUMENT, "tensor sizes overflow 64 bits");
    const uint64_t esz = in_dtype == KDA_BF16 ? 2 : 4;

    const uint64_t gsz = gate == kda::kGateLogitBf16 ? 2 : 4;
    const Span sp[] = {
        {"q", q, n_qk * esz}, {"k", k, n_qk * esz},    {"v", v, n_v * esz},         {"g", g, n_qk * gsz},
        {"beta", beta, n_tok * 4}, {"h0", h0, n_state * 4}, {"o", o, n_v * 4}, {"hT", hT, n_state * 4},
        {"ckpt", n_ckpt > 0 ? ckpt : nullptr, n_ck * 4},
    };
    constexpr int kO = 6, kHT = 7, kH0 = 5, kCk = 8;
    for (int i = 0; i < 8; ++i) {
        if (i != kO && overlaps(sp[kO], sp[i]))
            return fail(KDA_ERR_INVALID_ARGUMENT, "o overlaps %s", sp[i].name);
    }
    for (int i = 0; i < 5; ++i) {
        if (overlaps(sp[kHT], sp[i])) return fail(KDA_ERR_INVALID_ARGUMENT, "hT overlaps %s", sp[i].name);
    }
    if (overlaps(sp[kHT], sp[kH0]) && hT != h0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "hT partially overlaps h0 (only an exact alias is allowed)");
    for (int i = 0; i < 8; ++i) {
        if (overlaps(sp[kCk], sp[i])) return fail(KDA_ERR_INVALID_ARGUMENT, "ckpt overlaps %s", sp[i].name);
    }
    if (device_checks) {
        kda_status st = check_device();
        if (st != KDA_OK) return st;
        st = check_spans(sp, 9);
        if (st != KDA_OK) return st;
    }

    kda::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.o = o; a.hT = hT;
    a.gate = gate;
    a.g_min = g_min;
    a.ckpt = n_ckpt > 0 ? ckpt : nullptr;
    a.ckpt_every = ckpt ? ckpt_every / kda::kChunk : 0;
    a.n_ckpt = n_ckpt;
    a.B = B; a.T = T; a.H = H; a.D = static_cast<int>(Dk);
    a.bf16 = in_dtype == KDA_BF16;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(Dk));
    a.epoch = 0;
    a.qk_norm = qk_eps > 0.f;
    a.qk_eps2 = qk_eps * qk_eps;
    if (out) {
        *out = a;
        return ok();
    }
    if (T == 0 && !hT) return ok();  // nothing to compute or write
    return launch_prefill(a, static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *h0, float *o, float *hT, int64_t B, int64_t T, int64_t H, int64_t Dk,
                         int64_t Dv, kda_dtype in_dtype, float scale, void *stream) {
    return chunk_fwd(q, k, v, g, kda::kGateLogDecay, 0.f, beta, h0, o, hT, nullptr, 0, B, T, H, Dk, Dv, in_dtype,
                     scale, stream);
}

kda_status kda_chunk_fwd_ckpt(const void *q, const void *k, const void *v, const float *g, const float *beta,
                              const float *h0, float *o, float *hT, float *ckpt, int64_t ckpt_every, int64_t B,
                              int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale,
                              void *stream) {
    return chunk_fwd(q, k, v, g, kda::kGateLogDecay, 0.f, beta, h0, o, hT, ckpt, ckpt_every, B, T, H, Dk, Dv,
                     in_dtype, scale, stream, nullptr, true, 0.f, /*o_optional=*/true);
}

kda_status kda_chunk_fwd_gate(const void *q, const void *k, const void *v, const void *x, kda_dtype gate_dtype,
                              float g_min, const float *beta, const float *h0, float *o, float *hT, int64_t B,
                              int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale,
                              void *stream) {
    if (gate_dtype != KDA_F32 && gate_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown gate_dtype %d", static_cast<int>(gate_dtype));
    if (!(g_min >= -5.f && g_min < 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "g_min=%g must satisfy -5 <= g_min < 0", static_cast<double>(g_min));
    const kda::GateMode gate = gate_dtype == KDA_BF16 ? kda::kGateLogitBf16 : kda::kGateLogitF32;
    return chunk_fwd(q, k, v, x, gate, g_min, beta, h0, o, hT, nullptr, 0, B, T, H, Dk, Dv, in_dtype, scale,
                     stream);
}

kda_status kda_chunk_fwd_qknorm(const void *q, const void *k, const void *v, const void *g, kda_gate gate,
                                float g_min, float eps, const float *beta, const float *h0, float *o, float *hT,
                                int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype,
                                float scale, void *stream) {
    kda::GateMode mode;
    switch (gate) {
        case KDA_GATE_LOG_DECAY: mode = kda::kGateLogDecay; break;
        case KDA_GATE_LOGIT_F32: mode = kda::kGateLogitF32; break;
        case KDA_GATE_LOGIT_BF16: mode = kda::kGateLogitBf16; break;
        default: return fail(KDA_ERR_INVALID_ARGUMENT, "unknown gate kind %d", static_cast<int>(gate));
    }
    if (mode != kda::kGateLogDecay && !(g_min >= -5.f && g_min < 0.f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "g_min=%g must satisfy -5 <= g_min < 0", static_cast<double>(g_min));
    if (!(eps >= 1e-18f && eps <= 1e18f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "eps=%g must lie in [1e-18, 1e18]", static_cast<double>(eps));
    return chunk_fwd(q, k, v, g, mode, mode == kda::kGateLogDecay ? 0.f : g_min, beta, h0, o, hT, nullptr, 0, B, T,
                     H, Dk, Dv, in_dtype, scale, stream, nullptr, true, eps);
}

uint64_t kda_chunk_fwd_kcp_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t n_seg) {
    if (B <= 0 || T <= 0 || H <= 0 || Dk <= 0 || Dv <= 0 || n_seg <= 1 || T % n_seg != 0) return 0;
    uint64_t n = 3;
    if (!mul_ok(n, B) || !mul_ok(n, n_seg) || !mul_ok(n, H) || !mul_ok(n, Dk) || !mul_ok(n, Dv) || n > UINT64_MAX / 4)
        return 0;
    return n * 4;
}

}  // extern "C"

namespace {

// The segmented prefill.  `ws_fixed`: ws is the library's own per-device
// scratch array (kda_chunk_fwd_kcp_noalloc), already known to be a device
// buffer of ws_bytes that overlaps nothing; a request larger than it is
// rejected as unsupported.
kda_status chunk_fwd_kcp(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *h0, float *o, float *hT, int64_t n_seg, void *ws, uint64_t ws_bytes,
                         bool ws_fixed, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype,
                         float scale, void *stream) {
    if (n_seg < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "n_seg=%lld must be >= 1", (long long)n_seg);
    const bool split = n_seg > 1 && T > 0;
    uint64_t need = 0;
    if (split && B > 0 && H > 0 && Dk > 0 && Dv > 0) {  // (bad sizes are reported by the prefill checks)
        if (T % n_seg != 0)
            return fail(KDA_ERR_INVALID_ARGUMENT, "T=%lld is not a multiple of n_seg=%lld", (long long)T,
                        (long long)n_seg);
        need = kda_chunk_fwd_kcp_ws_bytes(B, T, H, Dk, Dv, n_seg);
        if (need == 0) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace size overflows 64 bits");
        if (ws_fixed && need > ws_bytes)
            return fail(KDA_ERR_UNSUPPORTED,
                        "the segmented prefill needs %llu bytes of workspace; the fixed array holds %llu "
                        "(3 * B * n_seg * H * Dk * Dv * 4 bytes must fit)",
                        (unsigned long long)need, (unsigned long long)ws_bytes);
        if (!ws || ws_bytes < need)
            return fail(KDA_ERR_INVALID_ARGUMENT, "ws (%llu bytes) must hold %llu bytes",
                        (unsigned long long)ws_bytes, (unsigned long long)need);
        if (!aligned16(ws)) return fail(KDA_ERR_INVALID_ARGUMENT, "ws is not 16-byte aligned");
    }
    kda::PrefillArgs a;
    kda_status st = chunk_fwd(q, k, v, g, kda::kGateLogDecay, 0.f, beta, h0, o, hT, nullptr, 0, B, T, H, Dk, Dv,
                              in_dtype, scale, stream, &a);
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!split) {
        if (T == 0 && !hT) return ok();
        return launch_prefill(a, s);
    }
    const uint64_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    const uint64_t n_tok = static_cast<uint64_t>(B) * T * H, n_state = static_cast<uint64_t>(B) * H * Dk * Dv;
    const Span wsp{"ws", ws, need};
    const Span others[] = {{"q", q, n_tok * Dk * esz}, {"k", k, n_tok * Dk * esz}, {"v", v, n_tok * Dv * esz},
                           {"g", g, n_tok * Dk * 4},   {"beta", beta, n_tok * 4},  {"h0", h0, n_state * 4},
                           {"o", o, n_tok * Dv * 4},   {"hT", hT, n_state * 4}};
    if (!ws_fixed) {
        for (const Span &x : others) {
            if (overlaps(wsp, x)) return fail(KDA_ERR_INVALID_ARGUMENT, "ws overlaps %s", x.name);
        }
        st = check_spans(&wsp, 1);
        if (st != KDA_OK) return st;
    }

    // segments as batch entries: [B, T, ...] is [B * n_seg, T / n_seg, ...]
    const int64_t L = T / n_seg, BP = B * n_seg;
    if (BP * H * 64 > INT32_MAX) return fail(KDA_ERR_UNSUPPORTED, "B*n_seg*H too large for one launch");
    const uint64_t per = static_cast<uint64_t>(BP) * H * Dk * Dv;  // floats of one set of segment states
    float *M = static_cast<float *>(ws), *Bs = M + per, *S_in = Bs + per;
    kda::PrefillArgs seg = a;
    seg.B = BP;
    seg.T = L;
    // pass 1: each segment from a zero state (its B_p), and from the identity
    // with zero values (its M_p); the outputs of these passes are not kept
    seg.h0 = nullptr;
    seg.hT = Bs;
    seg.o = nullptr;
    st = launch_prefill(seg, s);
    if (st != KDA_OK) return st;
    st = launch_status(kda::launch_fill_identity(S_in, BP * H, static_cast<int>(Dk), s), "kda identity fill");
    if (st != KDA_OK) return st;
    kda::PrefillArgs tr = seg;
    tr.v = nullptr;
    tr.h0 = S_in;
    tr.hT = M;
    st = launch_prefill(tr, s);
    if (st != KDA_OK) return st;
    // the incoming state of every segment, and the final state
    st = launch_status(kda::launch_kcp_combine(M, Bs, h0, S_in, hT, B, n_seg, H, static_cast<int>(Dk), s),
                       "kda segment combine");
    if (st != KDA_OK) return st;
    // pass 2: every segment from its incoming state, writing o
    kda::PrefillArgs fin = seg;
    fin.h0 = S_in;
    fin.hT = nullptr;
    fin.o = o;
    return launch_prefill(fin, s);
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_kcp(const void *q, const void *k, const void *v, const float *g, const float *beta,
                             const float *h0, float *o, float *hT, int64_t n_seg, void *ws, uint64_t ws_bytes,
                             int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale,
                             void *stream) {
    return chunk_fwd_kcp(q, k, v, g, beta, h0, o, hT, n_seg, ws, ws_bytes, false, B, T, H, Dk, Dv, in_dtype, scale,
                         stream);
}

kda_status kda_chunk_fwd_kcp_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                     const float *h0, float *o, float *hT, int64_t n_seg, int64_t B, int64_t T,
                                     int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale,
                                     void *stream) {
    // the device check comes first: the scratch lookup needs a usable current device
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    void *ws = nullptr;
    const hipError_t e = kda::kcp_scratch(&ws);
    if (e != hipSuccess) return fail(KDA_ERR_DEVICE, "scratch array lookup failed: %s", hipGetErrorString(e));
    return chunk_fwd_kcp(q, k, v, g, beta, h0, o, hT, n_seg, ws, kda::kKcpScratchBytes, true, B, T, H, Dk, Dv,
                         in_dtype, scale, stream);
}

uint64_t kda_chunk_fwd_kcp_noalloc_max_bytes(void) { return kda::kKcpScratchBytes; }

uint64_t kda_chunk_bwd_ws_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv) {
    if (B <= 0 || T < 0 || H <= 0 || Dk != Dv || (Dk != 16 && Dk != 128)) return 0;
    const int64_t ns = Dk == 128 ? 4 : 1;  // column slices of the backward kernel
    uint64_t ck = 1, pt = 1, tok = 1;
    if (!mul_ok(ck, T / kda::kChunk) || !mul_ok(ck, B) || !mul_ok(ck, H) || !mul_ok(ck, Dk) || !mul_ok(ck, Dv))
        return 0;
    if (!mul_ok(tok, B) || !mul_ok(tok, T) || !mul_ok(tok, H)) return 0;
    pt = tok;
    if (!mul_ok(pt, 3 * Dk + 1) || pt > UINT64_MAX - 3) return 0;
    pt = (pt + 3) / 4 * 4;  // each slice's partials start 16-byte aligned
    if (!mul_ok(pt, ns)) return 0;
    if (ck > UINT64_MAX / 8 || pt > UINT64_MAX / 8 || ck + pt > UINT64_MAX / 4) return 0;
    const uint64_t n = ck + pt;
    return n == 0 ? 16 : n * 4;
}

kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, const float *g, const float *beta,
                         const float *h0, const float *dO, const float *dhT, float *dq, float *dk, float *dv,
                         float *dg, float *dbeta, float *dh0, void *ws, uint64_t ws_bytes, int64_t B, int64_t T,
                         int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype, float scale, void *stream) {
    // the forward arguments are checked as for the prefill (with dq standing in for o;
    // the checkpoint pass itself writes no o)
    // (every host-side check comes before the device is queried)
    kda::PrefillArgs fa;
    kda_status st = chunk_fwd(q, k, v, g, kda::kGateLogDecay, 0.f, beta, h0, dq, nullptr, nullptr, 0, B, T, H, Dk, Dv,
                              in_dtype, scale, stream, &fa, false);
    if (st != KDA_OK) return st;
    if (T > 0 && (!dO || !dq || !dk || !dv || !dg || !dbeta))
        return fail(KDA_ERR_INVALID_ARGUMENT, "dO, dq, dk, dv, dg and dbeta must be non-null when T > 0");
    const uint64_t need = kda_chunk_bwd_ws_bytes(B, T, H, Dk, Dv);
    if (need == 0) return fail(KDA_ERR_INVALID_ARGUMENT, "workspace size overflows 64 bits");
    if (!ws || ws_bytes < need)
        return fail(KDA_ERR_INVALID_ARGUMENT, "ws (%llu bytes) must hold %llu bytes", (unsigned long long)ws_bytes,
                    (unsigned long long)need);
    const uint64_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    const uint64_t n_tok = static_cast<uint64_t>(B) * T * H, n_state = static_cast<uint64_t>(B) * H * Dk * Dv;
    const Span sp[] = {
        {"q", q, n_tok * Dk * esz}, {"k", k, n_tok * Dk * esz}, {"v", v, n_tok * Dv * esz},
        {"g", g, n_tok * Dk * 4},   {"beta", beta, n_tok * 4},  {"h0", h0, n_state * 4},
        {"dO", dO, n_tok * Dv * 4}, {"dhT", dhT, n_state * 4},  // inputs: 0 .. 7
        {"dq", dq, n_tok * Dk * 4}, {"dk", dk, n_tok * Dk * 4}, {"dv", dv, n_tok * Dv * 4},
        {"dg", dg, n_tok * Dk * 4}, {"dbeta", dbeta, n_tok * 4}, {"dh0", dh0, n_state * 4},
        {"ws", ws, need},  // outputs and workspace: 8 .. 14
    };
    constexpr int kN = 15, kFirstOut = 8;
    for (int i = kFirstOut; i < kN; ++i) {
        for (int j = 0; j < kN; ++j) {
            if (j != i && overlaps(sp[i], sp[j]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", sp[i].name, sp[j].name);
        }
    }
    st = check_device();
    if (st != KDA_OK) return st;
    st = check_spans(sp, kN);
    if (st != KDA_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *ckpt = static_cast<float *>(ws);
    const int64_t n_ck = T / kda::kChunk;
    // the states after every 16 tokens (a pass that writes no o)
    if (n_ck > 0) {
        kda::PrefillArgs ca = fa;
        ca.o = nullptr;
        ca.hT = nullptr;
        ca.ckpt = ckpt;
        ca.ckpt_every = 1;
        ca.n_ckpt = n_ck;
        st = launch_prefill(ca, s);
        if (st != KDA_OK) return st;
    }
    kda::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0; a.dO = dO; a.dhT = dhT; a.ckpt = ckpt;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.dh0 = dh0;
    a.part = ckpt + static_cast<uint64_t>(n_ck) * n_state;
    a.part_plane = static_cast<int64_t>(n_tok * Dk);
    a.part_stride = static_cast<int64_t>((n_tok * (3 * Dk + 1) + 3) / 4 * 4);  // as kda_chunk_bwd_ws_bytes
    a.B = B; a.T = T; a.H = H; a.D = static_cast<int>(Dk);
    a.bf16 = in_dtype == KDA_BF16;
    a.scale = fa.scale;
    if (T == 0 && !dh0) return ok();
    return launch_status(kda::launch_bwd(a, s), "kda backward");
}

}  // extern "C"

namespace {

// The decode entry points; qk_eps > 0 turns on the q/k normalisation.
kda_status decode_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                       float *state, float *o, int64_t B, int64_t H, int64_t Dk, int64_t Dv, kda_dtype in_dtype,
                       float scale, float qk_eps, void *stream) {
    if (B <= 0 || H <= 0 || Dk <= 0 || Dv <= 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "sizes must be positive: B=%lld H=%lld Dk=%lld Dv=%lld",
                    (long long)B, (long long)H, (long long)Dk, (long long)Dv);
    if (in_dtype != KDA_F32 && in_dtype != KDA_BF16)
        return fail(KDA_ERR_INVALID_ARGUMENT, "unknown in_dtype %d", static_cast<int>(in_dtype));
    if (Dk != Dv || (Dk != 16 && Dk != 128))
        return fail(KDA_ERR_UNSUPPORTED, "head dims Dk=%lld Dv=%lld: only Dk == Dv in {16, 128} is built",
                    (long long)Dk, (long long)Dv);
    if (!q || !k || !v || !g || !beta || !state || !o)
        return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be non-null");
    if (!std::isfinite(scale)) return fail(KDA_ERR_INVALID_ARGUMENT, "scale is not finite");
    uint64_t n_bh = 1, n_state = 1;
    if (!mul_ok(n_bh, B) || !mul_ok(n_bh, H) || !mul_ok(n_state, B) || !mul_ok(n_state, H) ||
        !mul_ok(n_state, Dk) || !mul_ok(n_state, Dv) || n_state > UINT64_MAX / 8)
        return fail(KDA_ERR_INVALID_ARGUMENT, "tensor sizes overflow 64 bits");
    if (n_bh > static_cast<uint64_t>(INT32_MAX)) return fail(KDA_ERR_UNSUPPORTED, "B*H too large for one launch");
    const uint64_t esz = in_dtype == KDA_BF16 ? 2 : 4;
    const Span sp[] = {
        {"q", q, n_bh * Dk * esz}, {"k", k, n_bh * Dk * esz}, {"v", v, n_bh * Dv * esz},
        {"g", g, n_bh * Dk * 4},   {"beta", beta, n_bh * 4},  {"state", state, n_state * 4},
        {"o", o, n_bh * Dv * 4},
    };
    for (int i = 0; i < 7; ++i) {
        for (int j = i + 1; j < 7; ++j) {
            const bool writes = (i >= 5 || j >= 5);
            if (writes && overlaps(sp[i], sp[j]))
                return fail(KDA_ERR_INVALID_ARGUMENT, "%s overlaps %s", sp[i].name, sp[j].name);
        }
    }
    kda_status st = check_device();
    if (st != KDA_OK) return st;
    st = check_spans(sp, 7);
    if (st != KDA_OK) return st;

    kda::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.o = o;
    a.B = B; a.H = H; a.D = static_cast<int>(Dk);
    a.bf16 = in_dtype == KDA_BF16;
    a.scale = scale > 0.f ? scale : 1.0f / std::sqrt(static_cast<float>(Dk));
    a.qk_norm = qk_eps > 0.f;
    a.qk_eps2 = qk_eps * qk_eps;
    return launch_status(kda::launch_decode(a, static_cast<hipStream_t>(stream)), "kda decode");
}

}  // namespace

extern "C" {

kda_status kda_decode_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           float *state, float *o, int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                           kda_dtype in_dtype, float scale, void *stream) {
    return decode_step(q, k, v, g, beta, state, o, B, H, Dk, Dv, in_dtype, scale, 0.f, stream);
}

kda_status kda_decode_step_qknorm(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                  float *state, float *o, int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                                  kda_dtype in_dtype, float scale, float eps, void *stream) {
    if (!(eps >= 1e-18f && eps <= 1e18f))
        return fail(KDA_ERR_INVALID_ARGUMENT, "eps=%g must lie in [1e-18, 1e18]", static_cast<double>(eps));
    return decode_step(q, k, v, g, beta, state, o, B, H, Dk, Dv, in_dtype, scale, eps, stream);
}

}  // extern "C"
