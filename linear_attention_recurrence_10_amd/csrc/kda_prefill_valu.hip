// kda_prefill_valu.hip -- chunked KDA prefill, fp32 arithmetic on the vector ALUs.
//
// This is the exact-precision path (fp32 products everywhere).  It serves fp32
// inputs (where the results must agree with the fp64 reference to ~1e-4) and
// head dimension 16; bf16 inputs at head dimension 128 go to the MFMA kernel.
//
// Chunk form (16-token chunks, one work-group per (batch, head, value-column
// slice)).  Within a chunk with start state S0 and per-channel cumulative
// log-decay gamma_r = g_1 + ... + g_r:
//   Qb = q * e^gamma, Kb = k * e^gamma, Kh = k * e^-gamma, Kd = k * e^(gamma_C - gamma)
//   A  = strict_lower(diag(beta) Kb Kh^T),  P = lower(Qb Kh^T)
//   (I + A) [W | Ut] = diag(beta) [Kb | V]            (forward substitution)
//   U  = Ut - W S0
//   O  = scale * (Qb S0 + P U)
//   S  = diag(e^gamma_C) S0 + Kd^T U
// This re-associates the token recurrence exactly: unrolling the decay of
// each key channel through the chunk turns the r-th write into a rank-1 term
// scaled by e^(gamma_C - gamma_r), and the coupled erase terms form the unit
// lower-triangular system above.  The chunk length 16 with gates >= -5 keeps
// e^(+-gamma) inside the normal fp32/bf16 range (Kimi K3 paper digest,
// devpress.csdn.net, section 2.1 (1)).
//
// With the q/k normalisation on, each staged q and k row is scaled by
// 1 / max(||x||, eps) before anything else reads it.
#include "kda_internal.h"

namespace kda {
namespace {

template <int D, int DVS, int RG, typename InT>
__global__ __launch_bounds__(DVS *RG) void prefill_valu_kernel(PrefillArgs a) {
    constexpr int NT = DVS * RG;
    constexpr int RPT = D / RG;  // state rows held per thread
    constexpr int NV = D / DVS;  // value-column slices per head
    constexpr int DP = D + 1;    // padded LDS row stride (bank-conflict free column reads)
    constexpr int C = kChunk;
    static_assert(D % RG == 0 && D % DVS == 0 && 64 % RG == 0, "bad tiling");

    __shared__ float sQ[C][DP];   // q, then Qb
    __shared__ float sKb[C][DP];  // Kb, then W
    __shared__ float sKh[C][DP];  // k, then Kh
    __shared__ float sKd[C][DP];  // Kd
    __shared__ float sG[C][DP];   // g, then gamma
    __shared__ float sV[C][DVS + 1];  // v slice, then Ut
    __shared__ float sA[C][C + 1];
    __shared__ float sP[C][C + 1];
    __shared__ float sBeta[C];
    __shared__ float sGC[D];  // e^gamma_C
    __shared__ float sNrm[2 * C];  // q/k normalisation factors [q rows, k rows]

    const int tid = threadIdx.x;
    const int c = tid / RG;   // value column inside the slice
    const int rg = tid % RG;  // row group: rows rg, rg+RG, ...
    int64_t blk = blockIdx.x;
    const int nv = static_cast<int>(blk % NV);
    blk /= NV;
    const int64_t h = blk % a.H;
    const int64_t b = blk / a.H;
    const int col = nv * DVS + c;
    const int64_t T = a.T, H = a.H;

    const InT *q = static_cast<const InT *>(a.q);
    const InT *k = static_cast<const InT *>(a.k);
    const InT *v = static_cast<const InT *>(a.v);

    const int64_t sbase = (b * H + h) * static_cast<int64_t>(D) * D;
    float S[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RG * m;
        S[m] = a.h0 ? a.h0[sbase + static_cast<int64_t>(i) * D + col] : 0.f;
    }

    const int64_t nchunks = (T + C - 1) / C;
    int64_t ck_left = a.ckpt_every, ck_i = 0;  // chunks to the next checkpoint, its index
    for (int64_t n = 0; n < nchunks; ++n) {
        const int64_t t0 = n * C;
        // (1) stage q, k, g (C x D), the value slice and beta; tokens past T are
        //     identity steps (g = 0, beta = 0, k = q = v = 0).
        for (int e = tid; e < C * D; e += NT) {
            const int r = e / D, i = e % D;
            const int64_t t = t0 + r;
            float qv = 0.f, kv = 0.f, gv = 0.f;
            if (t < T) {
                const int64_t idx = ((b * T + t) * H + h) * D + i;
                qv = ld_elem(q, idx);
                kv = ld_elem(k, idx);
                if (a.gate == kGateLogDecay)
                    gv = static_cast<const float *>(a.g)[idx];
                else if (a.gate == kGateLogitF32)
                    gv = gate_of_logit(static_cast<const float *>(a.g)[idx], a.g_min);
                else
                    gv = gate_of_logit(ld_elem(static_cast<const uint16_t *>(a.g), idx), a.g_min);
            }
            sQ[r][i] = qv;
            sKh[r][i] = kv;
            sG[r][i] = gv;
        }
        for (int e = tid; e < C * DVS; e += NT) {
            const int r = e / DVS, j = e % DVS;
            const int64_t t = t0 + r;
            sV[r][j] = (t < T && v) ? ld_elem(v, ((b * T + t) * H + h) * D + nv * DVS + j) : 0.f;
        }
        if (tid < C) {
            const int64_t t = t0 + tid;
            sBeta[tid] = (t < T) ? a.beta[(b * T + t) * H + h] : 0.f;
        }
        __syncthreads();

        // (1b) q/k normalisation (work-group uniform branch): one thread per
        //      row sums its squares, then every element is scaled
        if (a.qk_norm) {
            for (int rr = tid; rr < 2 * C; rr += NT) {
                const float *row = rr < C ? sQ[rr] : sKh[rr - C];
                float ss = 0.f;
                for (int i = 0; i < D; ++i) ss += row[i] * row[i];
                sNrm[rr] = norm_factor(ss, a.qk_eps2);
            }
            __syncthreads();
            for (int e = tid; e < C * D; e += NT) {
                const int r = e / D, i = e % D;
                sQ[r][i] *= sNrm[r];
                sKh[r][i] *= sNrm[C + r];
            }
            __syncthreads();
        }

        // (2) per-channel cumulative log-decay and the decay-scaled operands
        for (int i = tid; i < D; i += NT) {
            float gam = 0.f;
#pragma unroll
            for (int r = 0; r < C; ++r) {
                gam += sG[r][i];
                sG[r][i] = gam;
            }
            const float gC = gam;
            sGC[i] = expf(gC);
#pragma unroll
            for (int r = 0; r < C; ++r) {
                const float gr = sG[r][i];
                const float kv = sKh[r][i];
                const float e = expf(gr);
                sQ[r][i] *= e;
                sKb[r][i] = kv * e;
                sKh[r][i] = kv * expf(-gr);
                sKd[r][i] = kv * expf(gC - gr);
            }
        }
        __syncthreads();

        // (3) A = strict_lower(diag(beta) Kb Kh^T), P = lower(Qb Kh^T)
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            float accA = 0.f, accP = 0.f;
            if (s <= r) {
                for (int i = 0; i < D; ++i) {
                    const float kh = sKh[s][i];
                    accP += sQ[r][i] * kh;
                    accA += sKb[r][i] * kh;
                }
            }
            sA[r][s] = (s < r) ? sBeta[r] * accA : 0.f;
            sP[r][s] = (s <= r) ? accP : 0.f;
        }
        __syncthreads();

        // (4) (I + A) X = diag(beta) [Kb | V] by forward substitution, per column
        for (int j = tid; j < D + DVS; j += NT) {
            float x[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float y = sBeta[r] * (j < D ? sKb[r][j] : sV[r][j - D]);
#pragma unroll
                for (int s = 0; s < r; ++s) y -= sA[r][s] * x[s];
                x[r] = y;
            }
#pragma unroll
            for (int r = 0; r < C; ++r) {
                if (j < D)
                    sKb[r][j] = x[r];
                else
                    sV[r][j - D] = x[r];
            }
        }
        __syncthreads();

        // (5) U = Ut - W S0 and Qb S0 for this thread's column, reduced over the
        //     RG lanes that share the column (consecutive lanes of one wave)
        float u[C], qs[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float au = 0.f, aq = 0.f;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int i = rg + RG * m;
                au += sKb[r][i] * S[m];
                aq += sQ[r][i] * S[m];
            }
            u[r] = au;
            qs[r] = aq;
        }
#pragma unroll
        for (int off = 1; off < RG; off <<= 1) {
#pragma unroll
            for (int r = 0; r < C; ++r) {
                u[r] += __shfl_xor(u[r], off);
                qs[r] += __shfl_xor(qs[r], off);
            }
        }
#pragma unroll
        for (int r = 0; r < C; ++r) u[r] = sV[r][c] - u[r];

        // (6) O = scale * (Qb S0 + P U); lane rg stores rows r = rg (mod RG)
#pragma unroll
        for (int r = 0; r < C; ++r) {
            if ((r % RG) == rg && t0 + r < T && a.o) {
                float acc = qs[r];
#pragma unroll
                for (int s = 0; s <= r; ++s) acc += sP[r][s] * u[s];
                a.o[((b * T + t0 + r) * H + h) * D + col] = a.scale * acc;
            }
        }

        // (7) S = diag(e^gamma_C) S0 + Kd^T U
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            float acc = sGC[i] * S[m];
#pragma unroll
            for (int r = 0; r < C; ++r) acc += sKd[r][i] * u[r];
            S[m] = acc;
        }
        if (a.ckpt && --ck_left == 0) {  // the state after (ck_i + 1) * ckpt_every chunks
            if (ck_i < a.n_ckpt) {
                float *ck = a.ckpt + ck_i * (a.B * H * static_cast<int64_t>(D) * D) + sbase;
#pragma unroll
                for (int m = 0; m < RPT; ++m) ck[static_cast<int64_t>(rg + RG * m) * D + col] = S[m];
            }
            ++ck_i;
            ck_left = a.ckpt_every;
        }
        __syncthreads();  // LDS is reused by the next chunk
    }

    if (a.hT) {
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RG * m;
            a.hT[sbase + static_cast<int64_t>(i) * D + col] = S[m];
        }
    }
}

template <int D, int DVS, int RG>
hipError_t launch_d(const PrefillArgs &a, hipStream_t s) {
    const int64_t blocks = a.B * a.H * (D / DVS);
    dim3 grid(static_cast<unsigned>(blocks)), block(DVS * RG);
    if (a.bf16)
        hipLaunchKernelGGL((prefill_valu_kernel<D, DVS, RG, uint16_t>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((prefill_valu_kernel<D, DVS, RG, float>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_valu(const PrefillArgs &a, hipStream_t s) {
    switch (a.D) {
        case 16:
            return launch_d<16, 16, 4>(a, s);
        case 128:
            return launch_d<128, 32, 8>(a, s);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace kda
