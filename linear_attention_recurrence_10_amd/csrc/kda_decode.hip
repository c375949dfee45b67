// kda_decode.hip -- one-token KDA update of an fp32 state, in place.
//
// Per (batch, head), with a = e^g (per key channel) and S' = Diag(a) S:
//   r = S'^T k,  p = S'^T q,  e = beta (v - r)
//   S_new = S' + k e^T                       (written back over S)
//   o     = scale * S_new^T q = scale * (p + e (k . q))
// Decay first, then erase, then write ("Kimi K3 Architecture Explained",
// section 3 "Kimi Delta Attention (KDA)").  The state is read once and
// written once; everything else is a few hundred bytes per head, so the
// kernel is a streaming pass bounded by HBM bandwidth.
//
// Persistent work-groups walk the (batch, head) list with a stride of the
// grid size.  Thread (rg, jq) holds the float4 column quad jq of rows
// rg, rg + RG, ... of one state in registers; the next head's state is loaded
// while the current one is reduced and written back, so reads and writes of
// consecutive heads overlap.  The two column reductions (r, p) and k . q are
// combined across row groups through LDS.
//
// With the q/k normalisation (NORM), the sums of squares of q and k are
// combined the same way, and the factors c = 1 / max(||k||, eps) and
// d = 1 / max(||q||, eps) are applied where the raw vectors enter:
//   r = c S'^T k,  e = beta (v - r),  S_new = S' + k (c e)^T,
//   o = scale * d * (S'^T q + (c e) (k . q)).
#include <atomic>

#include "kda_internal.h"

namespace kda {
namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));

template <int D>
struct DecodeShape {
    static constexpr int NQ = D / 4;                                // float4 quads per row
    static constexpr int NT = (NQ * D < 512) ? NQ * D : 512;        // threads per work-group
    static constexpr int RG = NT / NQ;                              // row groups
    static constexpr int RPT = D / RG;                              // rows per thread
};

template <int D, typename InT, bool NORM>
__device__ __forceinline__ void decode_body(DecodeArgs a) {
    using Sh = DecodeShape<D>;
    constexpr int NQ = Sh::NQ, RG = Sh::RG, RPT = Sh::RPT;
    static_assert(RG * RPT == D && NQ * RG == Sh::NT, "bad decode tiling");

    __shared__ f32x4 sR[2][RG][NQ];
    __shared__ f32x4 sP[2][RG][NQ];
    __shared__ float sKQ[2][RG];
    __shared__ float sNrm[NORM ? 2 : 1][2][RG];  // sums of squares [par][q, k][row group]
    __shared__ f32x4 sE[2][NQ];

    const int tid = threadIdx.x;
    const int jq = tid % NQ;
    const int rg = tid / NQ;
    const int64_t BH = a.B * a.H;
    int64_t bh = blockIdx.x;
    if (bh >= BH) return;

    f32x4 s[RPT];
    {
        const f32x4 *S = reinterpret_cast<const f32x4 *>(a.state + bh * static_cast<int64_t>(D) * D);
#pragma unroll
        for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * NQ + jq]);
    }
    for (int par = 0; bh < BH; bh += gridDim.x, par ^= 1) {
        const int64_t nb = bh + gridDim.x;
        f32x4 sn[RPT];
        if (nb < BH) {  // next head's state, in flight while this head is processed
            const f32x4 *Sn = reinterpret_cast<const f32x4 *>(a.state + nb * static_cast<int64_t>(D) * D);
#pragma unroll
            for (int m = 0; m < RPT; ++m) sn[m] = __builtin_nontemporal_load(&Sn[(rg + RG * m) * NQ + jq]);
        }
        const InT *q = static_cast<const InT *>(a.q) + bh * D;
        const InT *k = static_cast<const InT *>(a.k) + bh * D;
        const InT *v = static_cast<const InT *>(a.v) + bh * D;
        const float *g = a.g + bh * D;
        f32x4 *S = reinterpret_cast<f32x4 *>(a.state + bh * static_cast<int64_t>(D) * D);

        float kk[RPT];
        f32x4 r4 = {0.f, 0.f, 0.f, 0.f}, p4 = r4;
        float kq = 0.f, qq = 0.f, k2 = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            const float ai = __expf(g[i]);
            const float ki = ld_elem(k, i);
            const float qi = ld_elem(q, i);
            kk[m] = ki;
            s[m] *= ai;
            r4 += ki * s[m];
            p4 += qi * s[m];
            kq += ki * qi;
            if constexpr (NORM) {
                qq += qi * qi;
                k2 += ki * ki;
            }
        }
        sR[par][rg][jq] = r4;
        sP[par][rg][jq] = p4;
        if (jq == 0) {
            sKQ[par][rg] = kq;
            if constexpr (NORM) {
                sNrm[par][0][rg] = qq;
                sNrm[par][1][rg] = k2;
            }
        }
        __syncthreads();

        if (rg == 0) {
            f32x4 rt = {0.f, 0.f, 0.f, 0.f}, pt = rt;
            float kqt = 0.f, qqt = 0.f, k2t = 0.f;
            for (int j = 0; j < RG; ++j) {
                rt += sR[par][j][jq];
                pt += sP[par][j][jq];
                kqt += sKQ[par][j];
                if constexpr (NORM) {
                    qqt += sNrm[par][0][j];
                    k2t += sNrm[par][1][j];
                }
            }
            const float bt = a.beta[bh];
            const int c0 = jq * 4;
            const f32x4 vv = {ld_elem(v, c0 + 0), ld_elem(v, c0 + 1), ld_elem(v, c0 + 2), ld_elem(v, c0 + 3)};
            if constexpr (NORM) {
                const float c = norm_factor(k2t, a.qk_eps2), d = norm_factor(qqt, a.qk_eps2);
                const f32x4 e = c * (bt * (vv - c * rt));  // c e: the write along the raw k
                sE[par][jq] = e;
                reinterpret_cast<f32x4 *>(a.o + bh * D)[jq] = (a.scale * d) * (pt + e * kqt);
            } else {
                const f32x4 e = bt * (vv - rt);
                sE[par][jq] = e;
                reinterpret_cast<f32x4 *>(a.o + bh * D)[jq] = a.scale * (pt + e * kqt);
            }
        }
        __syncthreads();

        const f32x4 e = sE[par][jq];
#pragma unroll
        for (int m = 0; m < RPT; ++m) __builtin_nontemporal_store(s[m] + kk[m] * e, &S[(rg + RG * m) * NQ + jq]);
        if (nb < BH) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) s[m] = sn[m];
        }
    }
}

template <int D, typename InT>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_kernel(DecodeArgs a) {
    decode_body<D, InT, false>(a);
}
// With the q/k normalisation (a kernel of its own name for kernel traces).
template <int D, typename InT>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_qknorm_kernel(DecodeArgs a) {
    decode_body<D, InT, true>(a);
}

// Work-groups resident at once: four per compute unit keeps enough state
// loads in flight to stream at close to the copy rate.
std::atomic<int> g_cus[64];

int decode_grid(int64_t BH) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    const int64_t g = static_cast<int64_t>(n) * 4;
    return static_cast<int>(BH < g ? BH : g);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(decode_grid(a.B * a.H))), block(DecodeShape<D>::NT);
    if (a.bf16 && a.qk_norm)
        hipLaunchKernelGGL((decode_qknorm_kernel<D, uint16_t>), grid, block, 0, s, a);
    else if (a.bf16)
        hipLaunchKernelGGL((decode_kernel<D, uint16_t>), grid, block, 0, s, a);
    else if (a.qk_norm)
        hipLaunchKernelGGL((decode_qknorm_kernel<D, float>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_kernel<D, float>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16:
            return launch_d<16>(a, s);
        case 128:
            return launch_d<128>(a, s);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace kda
