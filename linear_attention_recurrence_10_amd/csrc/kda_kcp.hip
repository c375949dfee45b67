// kda_kcp.hip -- the two small kernels of the segmented (sequence-parallel)
// prefill: an identity fill and the combine of the segments' affine maps.
//
// Splitting a sequence into P segments: the state after segment p is an
// affine function of the state before it, S_out = M_p S_in + B_p (the decays
// and erasures act on the key channels from the left; the writes add B_p).
// B_p is the segment's final state from a zero start, and M_p its final state
// from the identity with zero values.  This is the sequence split of the Kimi
// K3 paper digest (devpress.csdn.net), section 2.4 (1), where each GPU takes a
// segment and the states are exchanged once; here the segments are batch
// entries of one launch and the combine is a chain of P small products.
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

// The segmented prefill's workspace for callers that cannot allocate
// (kda_chunk_fwd_kcp_noalloc): one fixed array per device, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (on the
// host it is a stand-in symbol, not a device address); it uses the address
// hipGetSymbolAddress returns for the current device, kept per device below.
static __device__ __align__(256) unsigned char scratch[kKcpScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device ordinal; null until looked up

// states[n][D][D] = I
__global__ void fill_identity_kernel(float *states, int64_t n, int D) {
    const int64_t total = n * D * D;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int64_t r = (e / D) % D, c = e % D;
        states[e] = r == c ? 1.f : 0.f;
    }
}

// Work-group (b, h, cs) runs the chain for columns [CW cs, CW cs + CW) of the
// states (the columns are independent: S_{p+1}[:, j] = M_p S_p[:, j] + B_p[:, j]).
// Segment p's maps sit at batch entry b * P + p of the segment-batched states
// [B * P, H, D, D].  S_in[0] = h0 (or zeros), S_in[p] = M[p - 1] S_in[p - 1] +
// Bs[p - 1], hT = M[P - 1] S_in[P - 1] + Bs[P - 1].
//
// M[p] (all D x D) and the running column slice sit in LDS; each of the 256
// threads owns a TR x TC tile of the product, started from its tile of Bs[p].
// The next segment's M and Bs tile are loaded into registers while this
// segment's product runs.
template <int D, int NS>
__global__ __launch_bounds__(256) void combine_kernel(const float *M, const float *Bs, const float *h0, float *S_in,
                                                      float *hT, int64_t B, int64_t P, int64_t H) {
    constexpr int NT = 256, CW = D / NS;                    // columns per work-group
    constexpr int TC = CW >= 32 ? 4 : 1, TR = D * CW / (NT * TC);
    constexpr int LD = D + 4;                               // padded LDS row of M (keeps 16-byte rows)
    constexpr int ME = D * D / NT;                          // elements of M per thread
    constexpr int VW = ME % 4 == 0 ? 4 : 1;                 // loaded VW at a time
    static_assert(D % 4 == 0 && TR >= 1 && (D / TR) * (CW / TC) == NT && ME >= 1 && D * D % NT == 0, "tile shape");
    __shared__ __align__(16) float ms[D * LD];
    __shared__ __align__(16) float cur[D * CW];
    const int64_t bh = blockIdx.x / NS;
    const int cs = static_cast<int>(blockIdx.x % NS);
    const int64_t b = bh / H, h = bh % H;
    const int t = threadIdx.x;
    const int r0 = (t / (CW / TC)) * TR, c0 = (t % (CW / TC)) * TC;  // tile origin (column within the slice)
    const int col0 = cs * CW;
    auto at = [&](int64_t p) { return ((b * P + p) * H + h) * static_cast<int64_t>(D) * D; };
    const int64_t hb = bh * static_cast<int64_t>(D) * D;

    float mreg[ME];
    float breg[TR][TC];
    auto load_maps = [&](int64_t p) {
        const float *mp = M + at(p);
#pragma unroll
        for (int i = 0; i < ME / VW; ++i) {
            const int e = VW * (t + i * NT);
            if constexpr (VW == 4) {
                const float4 v = *reinterpret_cast<const float4 *>(mp + e);
                mreg[4 * i] = v.x;
                mreg[4 * i + 1] = v.y;
                mreg[4 * i + 2] = v.z;
                mreg[4 * i + 3] = v.w;
            } else {
                mreg[i] = mp[e];
            }
        }
        const float *bp = Bs + at(p);
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int j = 0; j < TC; ++j) breg[i][j] = bp[(r0 + i) * D + col0 + c0 + j];
    };
    auto store_m = [&]() {
#pragma unroll
        for (int i = 0; i < ME / VW; ++i) {
            const int e = VW * (t + i * NT);  // element of M: row e / D, columns e % D .. + VW - 1
#pragma unroll
            for (int j = 0; j < VW; ++j) ms[(e / D) * LD + e % D + j] = mreg[VW * i + j];
        }
    };

    for (int e = t; e < D * CW; e += NT) cur[e] = h0 ? h0[hb + (e / CW) * D + col0 + e % CW] : 0.f;
    load_maps(0);
    store_m();
    for (int64_t p = 0; p < P; ++p) {
        float acc[TR][TC];
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int j = 0; j < TC; ++j) acc[i][j] = breg[i][j];
        __syncthreads();  // ms holds M[p], cur holds S_p
        // this segment's incoming state
        float *sp = S_in + at(p);
        for (int e = t; e < D * CW; e += NT) sp[(e / CW) * D + col0 + e % CW] = cur[e];
        if (p + 1 < P) load_maps(p + 1);
        for (int k = 0; k < D; k += 4) {
            float a[TR][4], c[4][TC];
#pragma unroll
            for (int i = 0; i < TR; ++i)
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) a[i][kk] = ms[(r0 + i) * LD + k + kk];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int j = 0; j < TC; ++j) c[kk][j] = cur[(k + kk) * CW + c0 + j];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
#pragma unroll
                for (int i = 0; i < TR; ++i)
#pragma unroll
                    for (int j = 0; j < TC; ++j) acc[i][j] = __builtin_fmaf(a[i][kk], c[kk][j], acc[i][j]);
        }
        __syncthreads();  // every thread is done reading ms and cur
#pragma unroll
        for (int i = 0; i < TR; ++i)
#pragma unroll
            for (int j = 0; j < TC; ++j) cur[(r0 + i) * CW + c0 + j] = acc[i][j];
        if (p + 1 < P) store_m();
    }
    __syncthreads();
    if (hT) {
        for (int e = t; e < D * CW; e += NT) hT[hb + (e / CW) * D + col0 + e % CW] = cur[e];
    }
}

}  // namespace

hipError_t kcp_scratch(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

hipError_t launch_fill_identity(float *states, int64_t n, int D, hipStream_t s) {
    const int64_t total = n * D * D;
    const int64_t blocks = (total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096;
    hipLaunchKernelGGL(fill_identity_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, states, n, D);
    return hipGetLastError();
}

hipError_t launch_kcp_combine(const float *M, const float *Bs, const float *h0, float *S_in, float *hT, int64_t B,
                              int64_t P, int64_t H, int D, hipStream_t s) {
    if (D == 128)
        hipLaunchKernelGGL((combine_kernel<128, 4>), dim3(static_cast<unsigned>(B * H * 4)), dim3(256), 0, s, M, Bs,
                           h0, S_in, hT, B, P, H);
    else if (D == 16)
        hipLaunchKernelGGL((combine_kernel<16, 1>), dim3(static_cast<unsigned>(B * H)), dim3(256), 0, s, M, Bs, h0,
                           S_in, hT, B, P, H);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kda
