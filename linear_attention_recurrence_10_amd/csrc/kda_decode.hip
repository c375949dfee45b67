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
// One work-group per (batch, head).  Thread (rg, jq) holds the float4 column
// quad jq of rows rg, rg + RG, ... in registers; the two column reductions
// (r, p) and k . q are combined across row groups through LDS.
#include "kda_internal.h"

namespace kda {
namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));

template <int D>
struct DecodeShape {
    static constexpr int NQ = D / 4;                               // float4 quads per row
    static constexpr int NT = (NQ * D < 256) ? NQ * D : 256;       // threads per head
    static constexpr int RG = NT / NQ;                              // row groups
    static constexpr int RPT = D / RG;                              // rows per thread
};

template <int D, typename InT>
__global__ __launch_bounds__(DecodeShape<D>::NT) void decode_kernel(DecodeArgs a) {
    using Sh = DecodeShape<D>;
    constexpr int NQ = Sh::NQ, NT = Sh::NT, RG = Sh::RG, RPT = Sh::RPT;
    static_assert(RG * RPT == D && NQ * RG == NT, "bad decode tiling");

    __shared__ f32x4 sR[RG][NQ];
    __shared__ f32x4 sP[RG][NQ];
    __shared__ float sKQ[RG];
    __shared__ f32x4 sE[NQ];

    const int tid = threadIdx.x;
    const int jq = tid % NQ;
    const int rg = tid / NQ;
    const int64_t bh = blockIdx.x;

    const InT *q = static_cast<const InT *>(a.q) + bh * D;
    const InT *k = static_cast<const InT *>(a.k) + bh * D;
    const InT *v = static_cast<const InT *>(a.v) + bh * D;
    const float *g = a.g + bh * D;
    f32x4 *S = reinterpret_cast<f32x4 *>(a.state + bh * static_cast<int64_t>(D) * D);

    f32x4 s[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) s[m] = __builtin_nontemporal_load(&S[(rg + RG * m) * NQ + jq]);

    float kk[RPT];
    f32x4 r4 = {0.f, 0.f, 0.f, 0.f}, p4 = r4;
    float kq = 0.f;
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
    }
    sR[rg][jq] = r4;
    sP[rg][jq] = p4;
    if (jq == 0) sKQ[rg] = kq;
    __syncthreads();

    if (rg == 0) {
        f32x4 rt = {0.f, 0.f, 0.f, 0.f}, pt = rt;
        float kqt = 0.f;
        for (int j = 0; j < RG; ++j) {
            rt += sR[j][jq];
            pt += sP[j][jq];
            kqt += sKQ[j];
        }
        const float bt = a.beta[bh];
        const int c0 = jq * 4;
        const f32x4 vv = {ld_elem(v, c0 + 0), ld_elem(v, c0 + 1), ld_elem(v, c0 + 2), ld_elem(v, c0 + 3)};
        const f32x4 e = bt * (vv - rt);
        sE[jq] = e;
        reinterpret_cast<f32x4 *>(a.o + bh * D)[jq] = a.scale * (pt + e * kqt);
    }
    __syncthreads();

    const f32x4 e = sE[jq];
#pragma unroll
    for (int m = 0; m < RPT; ++m) __builtin_nontemporal_store(s[m] + kk[m] * e, &S[(rg + RG * m) * NQ + jq]);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DecodeShape<D>::NT);
    if (a.bf16)
        hipLaunchKernelGGL((decode_kernel<D, uint16_t>), grid, block, 0, s, a);
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
