// kda_bwd.hip -- gradient of the KDA forward pass (the training direction
// the FlashKDA kernel serves, Kimi K3 paper digest, devpress.csdn.net, section
// 2.4 (1)): the reverse-mode adjoint of the token recurrence
//   S'_t = Diag(exp g_t) S_{t-1},  r_t = S'_t^T k_t,  e_t = beta_t (v_t - r_t),
//   S_t = S'_t + k_t e_t^T,        o_t = scale S_t^T q_t,
// run from the last token to the first with dS = dL/dS_t:
//   dS += scale q_t do_t^T;  dq_t = scale S_t do_t;  de = dS^T k_t;  dk_t = dS e_t;
//   dbeta_t = de . (v_t - r_t);  dv_t = beta_t de;  dr = -beta_t de;
//   dS' = dS + k_t dr^T;  dk_t += S'_t dr;  dg_t = rowsum(dS' .* S'_t);  dS = Diag(exp g_t) dS'
// and dh0 = dS at the end.
//
// The forward states it needs come from state checkpoints every kBlk = 16
// tokens (written by the prefill kernels, one chunk apart).  Work-group
// (b, h, slice) owns columns [kCW slice, kCW slice + kCW) of the state, all
// Dk rows: the columns of S and dS are independent, so the slices of a head
// run side by side; what sums over columns (dq, dk, dg, dbeta) is written
// per slice and summed by a second kernel in a fixed order.  Inside a
// 16-token block the states are formed again from the checkpoint in fp32, in
// two halves of 8 tokens whose states stay in registers, and the adjoint runs
// over each half from its last token to its first.
//
// Lane layout: wave w of the work-group holds rows [kRW w, kRW w + kRW) of
// the slice; within it lane l holds the kRPL x kCPL tile of rows
// kRW w + kRPL (l / 8) + i and columns kCPL (l % 8) + j.  A sum over the
// columns of a row is a register sum plus shuffles among the 8 lanes of the
// row; a sum over the rows of a column is a register sum, shuffles among the
// 8 lanes of the column within the wave, and one exchange of the waves'
// partial sums through LDS.
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kBlk = 16;   // tokens between checkpoints
constexpr int kHalf = 8;   // tokens whose states are held in registers at a time

template <int D>
struct BwdShape;
template <>
struct BwdShape<128> {
    static constexpr int kCW = 32, kNW = 8;  // 32 columns per slice; 8 waves of 16 rows
};
template <>
struct BwdShape<16> {
    static constexpr int kCW = 16, kNW = 1;  // one slice; one wave of 16 rows
};

// x plus the value of another lane, moved by DPP (CTRL) or by a swizzle:
// quad_perm [1,0,3,2] is lane l ^ 1, quad_perm [2,3,0,1] lane l ^ 2 and
// row_ror:8 lane l ^ 8 (within each 16-lane row); the swizzle's bit mask
// 0x401f takes lane l ^ 16 (within each 32-lane half).
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float add_xor16(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
}
// row_shr:4 with out-of-row sources reading 0: lanes 4..7 of each group of 8
// add lanes 0..3
__device__ __forceinline__ float add_shr4(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, true));
}

__device__ __forceinline__ float ld_in(const void *p, int64_t i, bool bf16) {
    return bf16 ? ld_elem(static_cast<const uint16_t *>(p), i) : ld_elem(static_cast<const float *>(p), i);
}

template <int D, bool BF16>
__global__ __launch_bounds__(64 * BwdShape<D>::kNW) void bwd_kernel(BwdArgs a) {
    constexpr int kCW = BwdShape<D>::kCW, kNW = BwdShape<D>::kNW;
    constexpr int kNT = 64 * kNW;               // threads
    constexpr int kRW = D / kNW;                // rows per wave
    constexpr int kRPL = kRW / 8, kCPL = kCW / 8;  // rows and columns per lane
    constexpr int kNS = D / kCW;                // slices per head
    static_assert(kRPL * 8 == kRW && kCPL * 8 == kCW, "lane tiles");
    __shared__ float wsum[2][kNW][kCW];         // per-wave column sums (two buffers, used in turn)
    __shared__ float keep_r[kHalf][kCW], keep_e[kHalf][kCW];  // r_t, e_t of the half being reversed
    // the inputs of the 16-token block, staged with coalesced loads at its start
    __shared__ float s_k[kBlk][D], s_q[kBlk][D], s_a[kBlk][D];  // k, q, exp(g) by key channel
    __shared__ float s_v[kBlk][kCW], s_do[kBlk][kCW];          // v, dO of the slice's columns
    __shared__ float s_b[kBlk];                                 // beta

    const int64_t bh = blockIdx.x / kNS;
    const int slice = static_cast<int>(blockIdx.x % kNS);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r0 = w * kRW + (lane >> 3) * kRPL;  // first row of this lane
    const int c0 = (lane & 7) * kCPL;             // first column within the slice
    const int col0 = slice * kCW + c0;            // ... within the head
    const int64_t T = a.T, H = a.H;
    const int64_t sbase = bh * D * D + static_cast<int64_t>(r0) * D + col0;
    int par = 0;  // buffer of the next column sum

    // sums over all rows of the per-element values v[i][j]: out[j] for this lane's columns
    auto colsum = [&](const float (&v)[kRPL][kCPL], float (&out)[kCPL]) {
        float s[kCPL];
#pragma unroll
        for (int j = 0; j < kCPL; ++j) {
            s[j] = v[0][j];
#pragma unroll
            for (int i = 1; i < kRPL; ++i) s[j] += v[i][j];
            s[j] = add_dpp<0x128>(s[j]);  // + lane l ^ 8
            s[j] = add_xor16(s[j]);       // + lane l ^ 16
            s[j] += __shfl_xor(s[j], 32);
        }
        if constexpr (kNW == 1) {
#pragma unroll
            for (int j = 0; j < kCPL; ++j) out[j] = s[j];
        } else {
            if (lane < 8) {
#pragma unroll
                for (int j = 0; j < kCPL; ++j) wsum[par][w][c0 + j] = s[j];
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kCPL; ++j) {
                float t = wsum[par][0][c0 + j];
#pragma unroll
                for (int ww = 1; ww < kNW; ++ww) t += wsum[par][ww][c0 + j];
                out[j] = t;
            }
            par ^= 1;
        }
    };
    // sum over the slice's columns of a row (the 8 lanes with the same l / 8),
    // complete in the lanes with l % 8 >= 4 (kRowLane among them)
    auto rowsum = [&](float x) {
        x = add_dpp<0xb1>(x);  // + lane l ^ 1
        x = add_dpp<0x4e>(x);  // + lane l ^ 2
        return add_shr4(x);    // lanes 4..7 of each 8 add lanes 0..3
    };
    constexpr int kRowLane = 4;

    float dS[kRPL][kCPL];
#pragma unroll
    for (int i = 0; i < kRPL; ++i)
#pragma unroll
        for (int j = 0; j < kCPL; ++j) dS[i][j] = a.dhT ? a.dhT[sbase + i * D + j] : 0.f;

    const int64_t nblk = (T + kBlk - 1) / kBlk;
    const int64_t BHD = a.B * a.H * D * D;
    for (int64_t m = nblk - 1; m >= 0; --m) {
        const int64_t t0 = m * kBlk;
        const int64_t t1 = t0 + kBlk < T ? t0 + kBlk : T;
        // stage the block's inputs (tokens past the end are never read)
        __syncthreads();  // the previous block is done with the staged inputs
        const int nt = static_cast<int>(t1 - t0);
        for (int idx = tid; idx < kBlk * D; idx += kNT) {
            const int u = idx / D, c = idx % D;
            if (u < nt) {
                const int64_t o = ((b * T + t0 + u) * H + h) * D + c;
                s_k[u][c] = ld_in(a.k, o, BF16);
                s_q[u][c] = ld_in(a.q, o, BF16);
                s_a[u][c] = __expf(a.g[o]);
            }
        }
        for (int idx = tid; idx < kBlk * kCW; idx += kNT) {
            const int u = idx / kCW, c = idx % kCW;
            if (u < nt) {
                const int64_t o = ((b * T + t0 + u) * H + h) * D + slice * kCW + c;
                s_v[u][c] = ld_in(a.v, o, BF16);
                s_do[u][c] = a.dO[o];
            }
        }
        if (tid < nt) s_b[tid] = a.beta[(b * T + t0 + tid) * H + h];
        __syncthreads();
        float S0[kRPL][kCPL];  // the state before token t0
#pragma unroll
        for (int i = 0; i < kRPL; ++i)
#pragma unroll
            for (int j = 0; j < kCPL; ++j)
                S0[i][j] = m == 0 ? (a.h0 ? a.h0[sbase + i * D + j] : 0.f) : a.ckpt[(m - 1) * BHD + sbase + i * D + j];
        for (int half = 1; half >= 0; --half) {
            const int64_t u0 = t0 + half * kHalf;
            if (u0 >= t1) continue;
            const int nu = static_cast<int>(t1 - u0 < kHalf ? t1 - u0 : kHalf);
            float S[kRPL][kCPL];
#pragma unroll
            for (int i = 0; i < kRPL; ++i)
#pragma unroll
                for (int j = 0; j < kCPL; ++j) S[i][j] = S0[i][j];
            float st[kHalf][kRPL][kCPL];  // S_{t-1} of tokens u0 .. u0 + nu - 1
            // one forward token step on this lane's elements: S <- S_t
            auto fwd = [&](int ut, int u, bool keep) {
                float kk[kRPL], ai[kRPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    kk[i] = s_k[ut][r0 + i];
                    ai[i] = s_a[ut][r0 + i];
                }
                const float bt = s_b[ut];
                float sp[kRPL][kCPL], pr[kRPL][kCPL], r[kCPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i)
#pragma unroll
                    for (int j = 0; j < kCPL; ++j) {
                        sp[i][j] = ai[i] * S[i][j];
                        pr[i][j] = sp[i][j] * kk[i];
                    }
                colsum(pr, r);
#pragma unroll
                for (int j = 0; j < kCPL; ++j) {
                    const float e = bt * (s_v[ut][c0 + j] - r[j]);
#pragma unroll
                    for (int i = 0; i < kRPL; ++i) S[i][j] = sp[i][j] + kk[i] * e;
                    if (keep && tid < 8) {
                        keep_r[u][c0 + j] = r[j];
                        keep_e[u][c0 + j] = e;
                    }
                }
            };
            for (int ut = 0; ut < half * kHalf; ++ut) fwd(ut, 0, false);  // to the start of this half
#pragma unroll
            for (int u = 0; u < kHalf; ++u) {
                if (u < nu) {
#pragma unroll
                    for (int i = 0; i < kRPL; ++i)
#pragma unroll
                        for (int j = 0; j < kCPL; ++j) st[u][i][j] = S[i][j];
                    fwd(half * kHalf + u, u, true);
                }
            }
            __syncthreads();  // keep_r / keep_e of the half are visible
            // the adjoint over the half, last token first
#pragma unroll
            for (int u = kHalf - 1; u >= 0; --u) {
                if (u >= nu) continue;
                const int ut = half * kHalf + u;
                const int64_t rt = (b * T + u0 + u) * H + h;
                float kk[kRPL], qq[kRPL], ai[kRPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    kk[i] = s_k[ut][r0 + i];
                    qq[i] = s_q[ut][r0 + i];
                    ai[i] = s_a[ut][r0 + i];
                }
                const float bt = s_b[ut];
                float e[kCPL], rr[kCPL], dov[kCPL], vv[kCPL];
#pragma unroll
                for (int j = 0; j < kCPL; ++j) {
                    e[j] = keep_e[u][c0 + j];
                    rr[j] = keep_r[u][c0 + j];
                    dov[j] = s_do[ut][c0 + j];
                    vv[j] = s_v[ut][c0 + j];
                }
                float sp[kRPL][kCPL], pk[kRPL][kCPL];
                float sq[kRPL], se[kRPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    sq[i] = 0.f;
                    se[i] = 0.f;
#pragma unroll
                    for (int j = 0; j < kCPL; ++j) {
                        sp[i][j] = ai[i] * st[u][i][j];
                        // o_t = scale S_t^T q_t
                        dS[i][j] += a.scale * qq[i] * dov[j];
                        sq[i] += (sp[i][j] + kk[i] * e[j]) * dov[j];
                        // S_t = S'_t + k_t e_t^T
                        pk[i][j] = dS[i][j] * kk[i];
                        se[i] += dS[i][j] * e[j];
                    }
                }
                float de[kCPL];
                colsum(pk, de);
                // e_t = beta_t (v_t - r_t);  r_t = S'_t^T k_t;  S'_t = Diag(exp g_t) S_{t-1}
                float db = 0.f;
                float dr[kCPL];
#pragma unroll
                for (int j = 0; j < kCPL; ++j) {
                    db += de[j] * (vv[j] - rr[j]);
                    dr[j] = -bt * de[j];
                }
                float sdr[kRPL], sg[kRPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    sdr[i] = 0.f;
                    sg[i] = 0.f;
#pragma unroll
                    for (int j = 0; j < kCPL; ++j) {
                        const float dsp = dS[i][j] + kk[i] * dr[j];
                        sdr[i] += sp[i][j] * dr[j];
                        sg[i] += dsp * sp[i][j];
                        dS[i][j] = ai[i] * dsp;
                    }
                }
                float *part = a.part + static_cast<int64_t>(slice) * a.part_stride;
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    const float dq_i = a.scale * rowsum(sq[i]);
                    const float dk_i = rowsum(se[i] + sdr[i]);
                    const float dg_i = rowsum(sg[i]);
                    if ((lane & 7) == kRowLane) {
                        const int64_t o = rt * D + r0 + i;
                        part[o] = dq_i;
                        part[a.part_plane + o] = dk_i;
                        part[2 * a.part_plane + o] = dg_i;
                    }
                }
                const float dbs = rowsum(db);
                if (tid < 8) {
                    // dv_t: lanes 0..7 of wave 0 hold every column of the slice
#pragma unroll
                    for (int j = 0; j < kCPL; ++j) a.dv[rt * D + col0 + j] = bt * de[j];
                    if (tid == kRowLane) part[3 * a.part_plane + rt] = dbs;
                }
            }
            __syncthreads();  // keep_r / keep_e are rewritten by the next half
        }
    }
    if (a.dh0) {
#pragma unroll
        for (int i = 0; i < kRPL; ++i)
#pragma unroll
            for (int j = 0; j < kCPL; ++j) a.dh0[sbase + i * D + j] = dS[i][j];
    }
}

// The adjoint at Dk = Dv = 128 with a column per wave: work-group (b, h,
// slice) of 8 waves, wave w owns the slice's columns 4 w .. 4 w + 3 over all
// 128 rows, lane l rows 2 l and 2 l + 1.  A sum over the rows of a column
// (r_t, de) then stays inside one wave: a sum over each 16-lane row by DPP and
// four lane reads, the same value in every lane, with no barrier.  The
// forward steps that re-form the states of a block need only those sums, so
// all 16 states of a block are formed at once and kept in registers.  Sums
// over the columns of a row (dq, dk, dg) and over the columns (dbeta) are
// outputs that nothing waits for: each wave leaves its share of 8 tokens in
// LDS and they are summed over the waves once per 8 tokens.
template <int CTRL>
__device__ __forceinline__ float dpp_mv(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// the sum of x over all 64 lanes, in every lane (a fixed order: deterministic)
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_mv<0xb1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_mv<0x4e>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += dpp_mv<0x141>(x);  // row_half_mirror: the other quad of the 8
    x += dpp_mv<0x140>(x);  // row_mirror: the other 8 of the 16-lane row
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 48));
    return (r0 + r1) + (r2 + r3);
}

template <bool BF16>
__global__ __launch_bounds__(512) void bwd_col_kernel(BwdArgs a) {
    constexpr int D = 128, kCW = 32, kNW = 8, kCPW = kCW / kNW;  // 4 columns per wave
    constexpr int kRPL = 2;                                      // rows per lane
    constexpr int kNS = D / kCW;
    constexpr int kNQ = 3;  // sums over a row's columns: dq, dk, dg
    __shared__ float rowp[kHalf][kNQ][kNW][D];  // each wave's sums over its columns, 8 tokens
    __shared__ float dbp[kHalf][kNW];           // each wave's share of dbeta, 8 tokens
    __shared__ float keep_e[kBlk][kCW];         // e_t of the block, by column
    __shared__ float keep_r[kBlk][kCW];         // r_t of the block
    __shared__ float s_k[kBlk][D], s_q[kBlk][D], s_a[kBlk][D];
    __shared__ float s_v[kBlk][kCW], s_do[kBlk][kCW];
    __shared__ float s_b[kBlk];

    const int64_t bh = blockIdx.x / kNS;
    const int slice = static_cast<int>(blockIdx.x % kNS);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int r0 = kRPL * lane;                 // first row of this lane
    const int c0 = kCPW * w;                    // first column of this wave within the slice
    const int col0 = slice * kCW + c0;
    const int64_t T = a.T, H = a.H;
    const int64_t sbase = bh * D * D + static_cast<int64_t>(r0) * D + col0;
    float *part = a.part + static_cast<int64_t>(slice) * a.part_stride;

    float dS[kRPL][kCPW];
#pragma unroll
    for (int i = 0; i < kRPL; ++i)
#pragma unroll
        for (int j = 0; j < kCPW; ++j) dS[i][j] = a.dhT ? a.dhT[sbase + i * D + j] : 0.f;

    const int64_t nblk = (T + kBlk - 1) / kBlk;
    const int64_t BHD = a.B * a.H * D * D;
    for (int64_t m = nblk - 1; m >= 0; --m) {
        const int64_t t0 = m * kBlk;
        const int nt = static_cast<int>((t0 + kBlk < T ? t0 + kBlk : T) - t0);
        __syncthreads();  // the previous block is done with the staged inputs
        for (int idx = tid; idx < kBlk * D; idx += 512) {
            const int u = idx / D, c = idx % D;
            if (u < nt) {
                const int64_t o = ((b * T + t0 + u) * H + h) * D + c;
                s_k[u][c] = ld_in(a.k, o, BF16);
                s_q[u][c] = ld_in(a.q, o, BF16);
                s_a[u][c] = __expf(a.g[o]);
            }
        }
        for (int idx = tid; idx < kBlk * kCW; idx += 512) {
            const int u = idx / kCW, c = idx % kCW;
            if (u < nt) {
                const int64_t o = ((b * T + t0 + u) * H + h) * D + slice * kCW + c;
                s_v[u][c] = ld_in(a.v, o, BF16);
                s_do[u][c] = a.dO[o];
            }
        }
        if (tid < nt) s_b[tid] = a.beta[(b * T + t0 + tid) * H + h];
        __syncthreads();
        // the states before each token of the block, formed from the checkpoint
        float S[kRPL][kCPW];
#pragma unroll
        for (int i = 0; i < kRPL; ++i)
#pragma unroll
            for (int j = 0; j < kCPW; ++j)
                S[i][j] = m == 0 ? (a.h0 ? a.h0[sbase + i * D + j] : 0.f) : a.ckpt[(m - 1) * BHD + sbase + i * D + j];
        float st[kBlk][kRPL][kCPW];
#pragma unroll
        for (int u = 0; u < kBlk; ++u) {
            if (u < nt) {
                float kk[kRPL], ai[kRPL];
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    kk[i] = s_k[u][r0 + i];
                    ai[i] = s_a[u][r0 + i];
                }
                const float bt = s_b[u];
#pragma unroll
                for (int j = 0; j < kCPW; ++j) {
                    float pr = 0.f;
#pragma unroll
                    for (int i = 0; i < kRPL; ++i) {
                        st[u][i][j] = S[i][j];
                        S[i][j] *= ai[i];  // S'_t
                        pr += S[i][j] * kk[i];
                    }
                    const float r = wave_sum(pr);
                    const float e = bt * (s_v[u][c0 + j] - r);
#pragma unroll
                    for (int i = 0; i < kRPL; ++i) S[i][j] += kk[i] * e;
                    if (lane == 0) {
                        keep_e[u][c0 + j] = e;
                        keep_r[u][c0 + j] = r;
                    }
                }
            }
        }
        // (each wave reads only its own columns of keep_e / keep_r: no barrier needed)
        // the adjoint over the block, last token first; the sums over the
        // waves are taken after every 8 tokens
#pragma unroll
        for (int u = kBlk - 1; u >= 0; --u) {
            if (u >= nt) continue;
            const int64_t rt = (b * T + t0 + u) * H + h;
            const int us = u & (kHalf - 1);  // slot of the token in rowp / dbp
            float kk[kRPL], qq[kRPL], ai[kRPL];
#pragma unroll
            for (int i = 0; i < kRPL; ++i) {
                kk[i] = s_k[u][r0 + i];
                qq[i] = s_q[u][r0 + i];
                ai[i] = s_a[u][r0 + i];
            }
            const float bt = s_b[u];
            float sq[kRPL] = {}, se[kRPL] = {}, sdr[kRPL] = {}, sg[kRPL] = {};
            float dbw = 0.f;
#pragma unroll
            for (int j = 0; j < kCPW; ++j) {
                const float e = keep_e[u][c0 + j], rr = keep_r[u][c0 + j];
                const float dov = s_do[u][c0 + j], vv = s_v[u][c0 + j];
                float sp[kRPL], pk = 0.f;
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    sp[i] = ai[i] * st[u][i][j];
                    dS[i][j] += a.scale * qq[i] * dov;          // o_t = scale S_t^T q_t
                    sq[i] += (sp[i] + kk[i] * e) * dov;
                    pk += dS[i][j] * kk[i];                     // S_t = S'_t + k_t e_t^T
                    se[i] += dS[i][j] * e;
                }
                const float de = wave_sum(pk);
                dbw += de * (vv - rr);                          // e_t = beta_t (v_t - r_t)
                const float dr = -bt * de;
#pragma unroll
                for (int i = 0; i < kRPL; ++i) {
                    const float dsp = dS[i][j] + kk[i] * dr;    // r_t = S'_t^T k_t
                    sdr[i] += sp[i] * dr;
                    sg[i] += dsp * sp[i];                       // S'_t = Diag(exp g_t) S_{t-1}
                    dS[i][j] = ai[i] * dsp;
                }
                if (lane == 0) a.dv[rt * D + col0 + j] = bt * de;
            }
            // this wave's sums over its columns, to be summed over the waves
#pragma unroll
            for (int i = 0; i < kRPL; ++i) {
                rowp[us][0][w][r0 + i] = a.scale * sq[i];
                rowp[us][1][w][r0 + i] = se[i] + sdr[i];
                rowp[us][2][w][r0 + i] = sg[i];
            }
            if (lane == 0) dbp[us][w] = dbw;
            if (us == 0) {
                // tokens u .. min(u + 8, nt) - 1 of the block are done by every wave
                __syncthreads();
                const int n8 = nt - u < kHalf ? nt - u : kHalf;
                const int64_t rt0 = (b * T + t0 + u) * H + h;  // token u; token u + s is H rows later
                for (int idx = tid; idx < kNQ * D; idx += 512) {
                    const int q = idx / D, r = idx % D;
                    for (int s8 = 0; s8 < n8; ++s8) {
                        float x = rowp[s8][q][0][r];
#pragma unroll
                        for (int ww = 1; ww < kNW; ++ww) x += rowp[s8][q][ww][r];
                        part[q * a.part_plane + (rt0 + s8 * H) * D + r] = x;
                    }
                }
                if (tid < n8) {
                    float x = dbp[tid][0];
#pragma unroll
                    for (int ww = 1; ww < kNW; ++ww) x += dbp[tid][ww];
                    part[3 * a.part_plane + rt0 + tid * H] = x;
                }
                __syncthreads();  // rowp / dbp are written again by the next 8 tokens
            }
        }
    }
    if (a.dh0) {
#pragma unroll
        for (int i = 0; i < kRPL; ++i)
#pragma unroll
            for (int j = 0; j < kCPW; ++j) a.dh0[sbase + i * D + j] = dS[i][j];
    }
}

// A slice's partials are three planes of n_tok * D values (dq, dk, dg) and
// then n_tok values (dbeta).
__global__ void bwd_sum_kernel(const float *part, int64_t stride, int64_t plane, int ns, float *dq, float *dk,
                               float *dg, float *dbeta, int64_t n_tok) {
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < 3 * plane + n_tok;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        float s = 0.f;
        for (int sl = 0; sl < ns; ++sl) s += part[sl * stride + e];
        if (e < plane) dq[e] = s;
        else if (e < 2 * plane) dk[e - plane] = s;
        else if (e < 3 * plane) dg[e - 2 * plane] = s;
        else dbeta[e - 3 * plane] = s;
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    const int64_t BH = a.B * a.H;
    if (a.D == 128) {
        const dim3 grid(static_cast<unsigned>(BH * 4));
        if (a.bf16) hipLaunchKernelGGL((bwd_col_kernel<true>), grid, dim3(512), 0, s, a);
        else hipLaunchKernelGGL((bwd_col_kernel<false>), grid, dim3(512), 0, s, a);
    } else if (a.D == 16) {
        const dim3 grid(static_cast<unsigned>(BH));
        if (a.bf16) hipLaunchKernelGGL((bwd_kernel<16, true>), grid, dim3(64), 0, s, a);
        else hipLaunchKernelGGL((bwd_kernel<16, false>), grid, dim3(64), 0, s, a);
    } else {
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n_tok = a.B * a.T * a.H;
    const int64_t total = 3 * a.part_plane + n_tok;
    const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
    if (blocks > 0)
        hipLaunchKernelGGL(bwd_sum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a.part,
                           a.part_stride, a.part_plane, a.D == 128 ? 4 : 1, a.dq, a.dk, a.dg, a.dbeta, n_tok);
    return hipGetLastError();
}

}  // namespace kda
