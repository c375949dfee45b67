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
#include <type_traits>

#include "kda_f32mfma.h"

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

// ---- The chunk-form adjoint on the fp32 matrix cores (d = 128) ----
//
// The forward pass over a 16-token chunk with start state S0 (rows = key
// channels), per-channel cumulative log-decay gamma and D_C = diag(e^gamma_C):
//   Qb = q e^gamma, Kb = k e^gamma, Kh = k e^-gamma
//   A = strict_lower(diag(beta) Kb Kh^T),  N = (I + A)^-1,  M = N diag(beta)
//   P = lower(Qb Kh^T),  Z = V - Kb S0,  U = M Z
//   O = scale (Qb S0 + P U),  S = D_C (S0 + Kh^T U)
// is an exact regrouping of the token recurrence, so its adjoint is the
// gradient.  Given dS = dL/dS and the chunk's dO, with G = D_C dS:
//   dU = Kh G + scale P^T dO,  dZ = M^T dU  (= dv),  dM = dU Z^T,  dP = scale dO U^T
//   dS0 = G - Kb^T dZ + scale Qb^T dO                  (the next dS, one chunk back)
//   dN = dM diag(beta),  dA = -N^T dN N^T,  dGr = diag(beta) strict_lower(dA)
//   dbeta_s = sum_r dM_rs N_rs + sum_(u < s) dA_su (Kb Kh^T)_su
//   dQb = scale dO S0^T + dP Kh,  dKb = -dZ S0^T + dGr Kh,  dKh = U G^T + dGr^T Kb + dP^T Qb
//   dq = dQb e^gamma,  dk = dKb e^gamma + dKh e^-gamma
//   dgamma = dQb Qb + dKb Kb - dKh Kh,  plus rowsum(S .* dS) on gamma_C
//   dg_t = sum over u >= t of dgamma_u, plus the gamma_C term (every token of the chunk)
// In that last sum the pairs of tokens inside the chunk cancel except where
// they straddle t.  The pair of the state update (D_C Kh^T U, whose factor is
// e^(gamma_C - gamma_s)) is taken out of the cancellation: with W = (U G^T) .* Kh,
//   dg_t = sum_(u >= t) (dgamma_u + W_u) + rowsum(S0 .* G) + sum_(s < t) W_s,
// and so is the diagonal of P, whose pair has no decay factor at all: the
// products take dP without its diagonal, and the diagonal adds dP_tt k_t to
// dq_t and dP_tt q_t to dk_t directly.
// One work-group per (b, h, 32-column slice), eight waves.  The columns of S
// and dS are independent, so dS0, dZ and the slice's dv and dh0 are exact per
// slice; everything that sums over columns (dM, dP, the three d?b products
// and the gamma_C term) is linear in this slice's part, so each slice forms
// its share of dq, dk, dg and dbeta, and a second kernel sums the slices in a
// fixed order.  Every product is a 16 x 16 output tile of fp32 matrix-core
// instructions (16x16x4) with operands read from LDS; the phases of a chunk
// are separated by work-group barriers.  Waves w and w + 4 share a SIMD, so
// one wave's LDS and matrix-core latencies overlap the other's work.





// The inputs of one chunk for thread tid (wave w = tid / 64, lane l), in
// registers: token l % 16, channels 16 w + 4 (l / 16) .. + 3 of q, k (bf16)
// and g, so that each 16-lane row holds all 16 tokens of its 4 channels; v of
// the slice (token (tid % 64) / 4, columns 8 (tid % 4) ..); dO of the slice
// (with d = (tid - 64) % 128: token d / 8, columns 4 (d % 8) ..); the state
// before the chunk, rows tid / 8 and tid / 8 + 64, columns 4 (tid % 8) ..;
// beta of token tid % 16.
struct ChunkIn {
    uint2 q, k;
    uint4 v;
    float4 g, dO, s00, s01;
    float beta;
};


// tok0: row of token t0 of this (b, h) in [B, T, H] rows; nt: valid tokens
// of the chunk; s0: the state before the chunk (null: zero).
__device__ __forceinline__ ChunkIn load_chunk_inputs(const BwdArgs &a, int64_t tok0, int nt, int col0,
                                                     const float *s0, int64_t sb, int tid) {
    constexpr int D = 128;
    const uint32_t H = static_cast<uint32_t>(a.H), HD = H * D, last = static_cast<uint32_t>(nt - 1) * HD;
    const uint32_t off = static_cast<uint32_t>(tid & 15) * HD + 16 * (tid >> 6) + 4 * ((tid >> 4) & 3);  // elements
    const Rsrc rq = buf(static_cast<const uint16_t *>(a.q) + tok0 * D, 2 * (last + D));
    const Rsrc rk = buf(static_cast<const uint16_t *>(a.k) + tok0 * D, 2 * (last + D));
    const Rsrc rg = buf(a.g + tok0 * D, 4 * (last + D));
    const Rsrc rv = buf(static_cast<const uint16_t *>(a.v) + tok0 * D + col0, 2 * (last + 32));
    const Rsrc rd = buf(a.dO + tok0 * D + col0, 4 * (last + 32));
    const Rsrc rs = buf(s0 ? s0 + sb + col0 : nullptr, s0 ? 4u * (127 * D + 32) : 0u);
    const Rsrc rb = buf(a.beta + tok0, 4 * (static_cast<uint32_t>(nt - 1) * H + 1));
    ChunkIn in;
    in.q = ld8(rq, 2 * off);
    in.k = ld8(rk, 2 * off);
    in.g = ld16f(rg, 4 * off);
    // (v is stored by threads 0..63 and dO by threads 64..191, each thread the
    // piece it loads; the others load a piece too, to keep the loads free of
    // branches)
    const int l = tid & 63, l2 = (tid - 64) & 127;
    in.v = ld16(rv, 2 * (static_cast<uint32_t>(l >> 2) * HD + 8 * (l & 3)));
    in.dO = ld16f(rd, 4 * (static_cast<uint32_t>(l2 >> 3) * HD + 4 * (l2 & 7)));
    const uint32_t so = 4 * (static_cast<uint32_t>(tid >> 3) * D + 4 * (tid & 7));
    in.s00 = ld16f(rs, so);
    in.s01 = ld16f(rs, so + 4 * 64 * D);
    in.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (static_cast<uint32_t>(tid & 15) * H), 0, 0));
    return in;
}


template <int P, int PS>
__device__ __forceinline__ void put_row4(float (*sS0)[PS], float (*sS0T)[P], int c, int j, float4 x) {
    sS0[c][j] = x.x;
    sS0[c][j + 1] = x.y;
    sS0[c][j + 2] = x.z;
    sS0[c][j + 3] = x.w;
    sS0T[j][c] = x.x;
    sS0T[j + 1][c] = x.y;
    sS0T[j + 2][c] = x.z;
    sS0T[j + 3][c] = x.w;
}

// The chunk's inputs to LDS.  q, k and g become the operands at once: the
// cumulative log-decay gamma of each channel over the tokens (a prefix sum
// across the 16 lanes of a row, in token order), e^gamma and e^-gamma, Qb = q e^gamma,
// Kb = k e^gamma and Kh = k e^-gamma.  Tokens past the end were loaded as
// zeros, so they have zero operands and keep the last token's gamma.
template <int P, int PS>
__device__ __forceinline__ void store_chunk_inputs(const ChunkIn &in, int nt, int tid, float (*sQb)[P],
                                                   float (*sKb)[P], float (*sKh)[P], float (*sEg)[P],
                                                   float (*sEgi)[P], float (*sV)[PS], float (*sDO)[PS],
                                                   float (*sS0)[PS], float (*sS0T)[P], float *sBeta) {
    {
        const int t = tid & 15, c0 = 16 * (tid >> 6) + 4 * ((tid >> 4) & 3);
        float gam[4] = {in.g.x, in.g.y, in.g.z, in.g.w};
        // prefix sums over the 16 tokens of the row, summed in token order:
        // fifteen rounds of "the previous lane's sum plus my g" (the lane before
        // the row's start reads 0) leave lane t with ((g_0 + g_1) + ...) + g_t.
        // A log-depth scan rounds gamma_t and gamma_(t-1) independently; this
        // order keeps their difference g_t up to one rounding, which the
        // decay ratios e^(gamma_t - gamma_s) of the gradient need (with the
        // log-depth scan the largest dg error on the B=4 H=16 T=4096 workload
        // was 2.8 times as large)
        {
            const float g0[4] = {gam[0], gam[1], gam[2], gam[3]};
#pragma unroll
            for (int st = 1; st < 16; ++st) {
#pragma unroll
                for (int j = 0; j < 4; ++j) gam[j] = dpp_mv<0x111>(gam[j]) + g0[j];  // row_shr:1
            }
        }
        const uint32_t qw[2] = {in.q.x, in.q.y}, kw[2] = {in.k.x, in.k.y};
        f32x4 qb, kb, kh, eg, egi;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float e = __expf(gam[j]), ei = __expf(-gam[j]);
            const float qv = (j & 1) ? bf_hi(qw[j >> 1]) : bf_lo(qw[j >> 1]);
            const float kv = (j & 1) ? bf_hi(kw[j >> 1]) : bf_lo(kw[j >> 1]);
            qb[j] = qv * e;
            kb[j] = kv * e;
            kh[j] = kv * ei;
            eg[j] = e;
            egi[j] = ei;
        }
        *reinterpret_cast<f32x4 *>(&sQb[t][c0]) = qb;
        *reinterpret_cast<f32x4 *>(&sKb[t][c0]) = kb;
        *reinterpret_cast<f32x4 *>(&sKh[t][c0]) = kh;
        *reinterpret_cast<f32x4 *>(&sEg[t][c0]) = eg;
        *reinterpret_cast<f32x4 *>(&sEgi[t][c0]) = egi;
    }
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (wv == 0) {
        const int vt = tid >> 2, vc = 8 * (tid & 3);
        const bool vl = vt < nt;
        sV[vt][vc + 0] = vl ? bf_lo(in.v.x) : 0.f;
        sV[vt][vc + 1] = vl ? bf_hi(in.v.x) : 0.f;
        sV[vt][vc + 2] = vl ? bf_lo(in.v.y) : 0.f;
        sV[vt][vc + 3] = vl ? bf_hi(in.v.y) : 0.f;
        sV[vt][vc + 4] = vl ? bf_lo(in.v.z) : 0.f;
        sV[vt][vc + 5] = vl ? bf_hi(in.v.z) : 0.f;
        sV[vt][vc + 6] = vl ? bf_lo(in.v.w) : 0.f;
        sV[vt][vc + 7] = vl ? bf_hi(in.v.w) : 0.f;
    } else if (wv < 3) {
        const int dt = (tid - 64) >> 3, dc = 4 * ((tid - 64) & 7);
        const bool dl = dt < nt;
        sDO[dt][dc] = dl ? in.dO.x : 0.f;
        sDO[dt][dc + 1] = dl ? in.dO.y : 0.f;
        sDO[dt][dc + 2] = dl ? in.dO.z : 0.f;
        sDO[dt][dc + 3] = dl ? in.dO.w : 0.f;
    }
    const int r0 = tid >> 3, j = 4 * (tid & 7);
    put_row4(sS0, sS0T, r0, j, in.s00);
    put_row4(sS0, sS0T, r0 + 64, j, in.s01);
    if (tid < 16) sBeta[tid] = tid < nt ? in.beta : 0.f;
}


// bf16 inputs (fp32 inputs take the token-serial kernel).
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdArgs a) {
    constexpr int D = 128, kCW = 32, kNS = D / kCW, kC = 16;
    constexpr int kP = 132;  // pitch of the token x channel arrays
    constexpr int kPS = 36;  // pitch of the channel x column and token x column arrays
    constexpr int kP16 = 20; // pitch of the 16 x 16 arrays
    __shared__ float sQb[kC][kP], sKb[kC][kP], sKh[kC][kP], sEg[kC][kP], sEgi[kC][kP], sDgam[kC][kP], sW[kC][kP];
    __shared__ float sS0[D][kPS], sG[D][kPS];
    __shared__ float sS0T[kCW][kP], sGT[kCW][kP];  // transposed copies: column j, channel c
    __shared__ float sV[kC][kPS], sDO[kC][kPS], sZ[kC][kPS], sU[kC][kPS], sdU[4][kC][kPS], sdZ[kC][kPS];
    __shared__ float sA[kC][kP16], sGr[kC][kP16], sPs[kC][kP16], sN[kC][kP16], sM[kC][kP16];
    __shared__ float sdP[kC][kP16], sdGr[kC][kP16];
    __shared__ float sBeta[kC], sDgC[D], sDB[kC], sDPd[kC];

    const int64_t bh = blockIdx.x / kNS;
    const int slice = static_cast<int>(blockIdx.x % kNS);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid_k = threadIdx.x, tid = tid_k, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
    // wave-uniform: its branches and offsets are scalar.  Wave w owns row
    // block w of dS (channels 16 w .. 16 w + 15, both column tiles) and
    // channel block w of the d?b products.
    const int w = __builtin_amdgcn_readfirstlane(tid_k >> 6);
    const int64_t T = a.T, H = a.H;
    const int col0 = slice * kCW;
    float *part = a.part + static_cast<int64_t>(slice) * a.part_stride;
    const int64_t BHD = a.B * a.H * D * D;
    const int64_t sb = bh * D * D;
    const uint32_t HD = static_cast<uint32_t>(a.H) * D;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // dS, this wave's two tiles of the 128 x 32 slice: tile ct is row block w,
    // column tile ct; component i is row 4 g4 + i of the block
    f32x4 dS[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            dS[ct][i] = a.dhT ? a.dhT[sb + (16 * w + 4 * g4 + i) * D + col0 + 16 * ct + r16] : 0.f;
    }
    // (dS has landed before the loop: without this wait the loop would wait for
    // every outstanding store, once per chunk, where it first scales dS)
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)

    const int64_t nch = (T + kC - 1) / kC;
    ChunkIn in{};
    if (nch > 0) {
        const int64_t t0 = (nch - 1) * kC;
        in = load_chunk_inputs(a, (b * T + t0) * H + h, static_cast<int>(T - t0), col0,
                               nch - 1 == 0 ? a.h0 : a.ckpt + (nch - 2) * BHD, sb, tid);  // (the last chunk)
    }
    for (int64_t n = nch - 1; n >= 0; --n) {
        const int64_t t0 = n * kC;
        const int nt = static_cast<int>(t0 + kC < T ? kC : T - t0);
        // The lane's indices, made opaque to the compiler once per chunk: the
        // LDS addresses of the chunk are then formed in the loop from a few
        // registers instead of being kept, one register each, across it.
        int tidv = tid_k;
        asm volatile("" : "+v"(tidv));
        const int tid = tidv, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
        // this chunk's outputs: wave-uniform bases at token t0 plus 32-bit lane offsets
        const int64_t tok0 = (b * T + t0) * H + h;
        const uint32_t last = static_cast<uint32_t>(nt - 1) * HD;
        const Rsrc dvb = buf(a.dv + tok0 * D + col0, 4 * (last + 32));
        const Rsrc pq = buf(part + tok0 * D, 4 * (last + D));
        const Rsrc pk = buf(part + a.part_plane + tok0 * D, 4 * (last + D));
        const Rsrc pg = buf(part + 2 * a.part_plane + tok0 * D, 4 * (last + D));
        const Rsrc pb = buf(part + 3 * a.part_plane + tok0, 4 * (static_cast<uint32_t>(nt - 1) * static_cast<uint32_t>(H) + 1));
        // (no barrier here: the dg pass of the previous chunk reads only sDgam,
        // sW, sDgC and sDB, which the store below leaves alone, and the barrier
        // before that pass already ordered B4's reads of the operands)

        // (L) the chunk's inputs, loaded during the previous chunk (or before
        //     the loop), to LDS: the decay factors and the scaled operands
        //     Qb, Kb, Kh are formed on the way (e^gamma_C is row 15 of sEg)
        store_chunk_inputs(in, nt, tid, sQb, sKb, sKh, sEg, sEgi, sV, sDO, sS0, sS0T, sBeta);
        lds_barrier();
        // (F1) Kb Kh^T and A (wave 0), scale P (wave 1), Z = V - Kb S0 (waves 2,
        // 3); waves 4 .. 7 start their dQb tiles: dO S0^T (transposed: channel
        // block w as rows).  Waves 0 .. 3 start theirs in F3.
        f32x4 accQ = zero, accKb, accKh;
        if (w == 0) {
            const f32x4 gr = tile_mm_kc<D>(&sKb[0][0], kP, &sKh[0][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                sGr[r][r16] = gr[i];
                sA[r][r16] = r16 < r ? sBeta[r] * gr[i] : 0.f;
            }
        } else if (w == 1) {
            const f32x4 pr = tile_mm_kc<D>(&sQb[0][0], kP, &sKh[0][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                sPs[r][r16] = r16 <= r ? a.scale * pr[i] : 0.f;
            }
        } else if (w < 4) {
            const int ct = w - 2;
            const f32x4 x = tile_mm_kc<D>(&sKb[0][0], kP, &sS0T[16 * ct][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g4 + i;
                sZ[t][16 * ct + r16] = sV[t][16 * ct + r16] - x[i];
            }
        } else {
            accQ = tile_mm_kc<kCW>(&sS0[16 * w][0], kPS, &sDO[0][0], kPS, zero, lane);
        }
        lds_barrier();

        // (F2) N = (I + A)^-1 and M = N diag(beta): row group g4 of wave w < 4
        // solves column 4 w + g4
        if (w < 4) {
            float nar[kC];
#pragma unroll
            for (int u = 0; u < kC; ++u) nar[u] = -sA[r16][u];
            const int s = 4 * w + g4;
            float x = r16 == s ? 1.f : 0.f;
            solve_pivots<0>(x, nar);
            sN[r16][s] = x;
            sM[r16][s] = x * sBeta[s];
        }
        lds_barrier();

        // (F3) U = M Z (waves 0, 1); waves 0 .. 3 start their dQb tiles
        if (w < 2) {
            const f32x4 uu = tile_mm<kC>(&sM[0][0], kP16, 1, &sZ[0][16 * w], kPS, 1, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sU[4 * g4 + i][16 * w + r16] = uu[i];
        }
        if (w < 4) accQ = tile_mm_kc<kCW>(&sS0[16 * w][0], kPS, &sDO[0][0], kPS, zero, lane);

        // (F4) G = D_C dS (kept in dS and written for the products) and the
        // gamma_C term of D_C S0: rowsum(S0 .* G)
        {
            f32x4 dgc = zero;
            // (rows 4 g4 .. 4 g4 + 3 of a tile are consecutive in sEg's last row,
            // in sS0T and in sGT: one 16-byte access each)
            const int row0 = 16 * w + 4 * g4;
            const f32x4 egc = *reinterpret_cast<const f32x4 *>(&sEg[kC - 1][row0]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int col = 16 * ct + r16;
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(&sS0T[col][row0]);
                dS[ct] *= egc;
                dgc += s0 * dS[ct];
#pragma unroll
                for (int i = 0; i < 4; ++i) sG[row0 + i][col] = dS[ct][i];
                *reinterpret_cast<f32x4 *>(&sGT[col][row0]) = dS[ct];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = row_sum16(dgc[i]);
                if (r16 == 0) sDgC[row0 + i] = v;
            }
        }
        lds_barrier();

        // (B1) dU = Kh G + scale P^T dO in four channel quarters (wave w: column
        // tile w % 2, quarter w / 2); dKh starts as U G^T; wave 7 forms dP
        {
            const int ct = w & 1, kq = w >> 1;
            f32x4 du = tile_mm_kc<32>(&sKh[0][32 * kq], kP, &sGT[16 * ct][32 * kq], kP, zero, lane);
            if (kq == 0) du = tile_mm<kC>(&sPs[0][0], 1, kP16, &sDO[0][16 * ct], kPS, 1, du, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sdU[kq][4 * g4 + i][16 * ct + r16] = du[i];
        }
        accKh = tile_mm_kc<kCW>(&sG[16 * w][0], kPS, &sU[0][0], kPS, zero, lane);
        if (w == 7) {
            const f32x4 dp = tile_mm_kc<kCW>(&sDO[0][0], kPS, &sU[0][0], kPS, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                sdP[r][r16] = r16 < r ? a.scale * dp[i] : 0.f;
                if (r16 == r) sDPd[r] = a.scale * dp[i];
            }
        }
        lds_barrier();

        // (B2) dZ = M^T dU (waves 0, 1; it is dv); dM = dU Z^T and the solve's
        // adjoint (wave 3).  dU is the sum of B1's four quarters.
        if (w < 2) {
            const int ct = w;
            f32x4 dz = zero;
#pragma unroll
            for (int k0 = 0; k0 < kC; k0 += 4) {
                const int k = k0 + g4, c = 16 * ct + r16;
                dz = mfma4(sM[k][r16], (sdU[0][k][c] + sdU[1][k][c]) + (sdU[2][k][c] + sdU[3][k][c]), dz);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g4 + i;
                sdZ[t][16 * ct + r16] = dz[i];
                st4(dvb, 4 * (static_cast<uint32_t>(t) * HD + 16 * ct + r16), dz[i]);
            }
        } else if (w == 3) {
            // dM^T = Z dU^T, then back through the solve: T1 = dN N^T with
            // dN = dM diag(beta), dA = -N^T T1, dGr and this slice's dbeta.
            // Each product's result feeds the next one from registers: lane
            // (r16, g4) holds rows 4 g4 + i of column r16 of a result, which
            // are that lane's operand values when the next product takes
            // k = 4 g4 + m at step m (the order of a sum over k is free).
            f32x4 dmt = zero;  // lane (r16, g4): dM(r16, 4 g4 + i)
#pragma unroll
            for (int k0 = 0; k0 < kCW; k0 += 4) {
                const int k = k0 + g4;
                dmt = mfma4(sZ[r16][k], (sdU[0][r16][k] + sdU[1][r16][k]) + (sdU[2][r16][k] + sdU[3][r16][k]), dmt);
            }
            f32x4 t1 = zero;  // T1(4 g4 + i, r16) = sum_s dM(4 g4 + i, s) beta_s N(r16, s)
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int sk = 4 * g4 + m;
                t1 = mfma4(dmt[m] * sBeta[sk], sN[r16][sk], t1);
            }
            f32x4 na = zero;  // (N^T T1)(4 g4 + i, r16)
#pragma unroll
            for (int m = 0; m < 4; ++m) na = mfma4(sN[4 * g4 + m][r16], t1[m], na);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                const float da = r16 < r ? -na[i] : 0.f;
                sdGr[r][r16] = sBeta[r] * da;
                // dbeta_r = sum over rows u of dM_ur N_ur (column r of dM .* N) plus
                // sum over s < r of dA_rs (Kb Kh^T)_rs (row r of dA .* Gr)
                const float db = row_sum16(dmt[i] * sN[r16][r]) + row_sum16(da * sGr[r][r16]);
                if (r16 == 0) sDB[r] = db;
            }
        }
        lds_barrier();

        // the next chunk's loads, issued among the products of B3 (straight-line
        // code in every wave), are in flight through B4 and the dg pass (in the
        // last step, chunk 0 again: the loads are the same every step)
        {
            const int64_t np = n > 0 ? n - 1 : 0;
            in = load_chunk_inputs(a, (b * T + np * kC) * H + h, n > 0 ? kC : nt, col0,
                                   np == 0 ? a.h0 : a.ckpt + (np - 1) * BHD, sb, tid);
        }
        // (B3) dS0 = G - Kb^T dZ + scale Qb^T dO (this wave's tiles: the next
        // dS); dKb starts as -dZ S0^T
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const f32x4 t1 = tile_mm<kC>(&sKb[0][16 * w], 1, kP, &sdZ[0][16 * ct], kPS, 1, zero, lane);
            const f32x4 t2 = tile_mm<kC>(&sQb[0][16 * w], 1, kP, &sDO[0][16 * ct], kPS, 1, zero, lane);
            dS[ct] = (dS[ct] - t1) + a.scale * t2;
        }
        accKb = tile_mm_kc<kCW>(&sS0[16 * w][0], kPS, &sdZ[0][0], kPS, zero, lane);
        // (B3 writes no LDS: B4 follows without a barrier)

        // (B4) finish dQb, dKb, dKh on this wave's channel block; dq, dk and
        // dgamma of its 16 tokens x 16 channels.  The tiles are transposed
        // (channel rows, token columns; the accumulators above likewise), so
        // lane (r16, g4) holds channels 4 g4 .. 4 g4 + 3 of token r16: its LDS
        // reads and writes and its partial stores are 16 bytes each.
        {
            const int cb = w;
            f32x4 dqb = a.scale * accQ;
            dqb = tile_mm<kC>(&sKh[0][16 * cb], 1, kP, &sdP[0][0], 1, kP16, dqb, lane);
            f32x4 dkb = -accKb;
            dkb = tile_mm<kC>(&sKh[0][16 * cb], 1, kP, &sdGr[0][0], 1, kP16, dkb, lane);
            // the pairs' part of dKh on its own (the U G^T part is W, summed apart)
            f32x4 dkh = tile_mm<kC>(&sKb[0][16 * cb], 1, kP, &sdGr[0][0], kP16, 1, zero, lane);
            dkh = tile_mm<kC>(&sQb[0][16 * cb], 1, kP, &sdP[0][0], kP16, 1, dkh, lane);
            const int t = r16, c = 16 * cb + 4 * g4;
            const f32x4 eg = *reinterpret_cast<const f32x4 *>(&sEg[t][c]);
            const f32x4 egi = *reinterpret_cast<const f32x4 *>(&sEgi[t][c]);
            const f32x4 kh = *reinterpret_cast<const f32x4 *>(&sKh[t][c]);
            const f32x4 qb = *reinterpret_cast<const f32x4 *>(&sQb[t][c]);
            const f32x4 kb = *reinterpret_cast<const f32x4 *>(&sKb[t][c]);
            const float dpd = sDPd[t];
            *reinterpret_cast<f32x4 *>(&sDgam[t][c]) = (dqb * qb + dkb * kb) - dkh * kh;
            *reinterpret_cast<f32x4 *>(&sW[t][c]) = accKh * kh;
            const uint32_t o = 4 * (static_cast<uint32_t>(t) * HD + c);
            st16(pq, o, dqb * eg + dpd * (kb * egi));                        // + dP_tt k_t
            st16(pk, o, (dkb * eg + (accKh + dkh) * egi) + dpd * (qb * egi));  // + dP_tt q_t
        }
        lds_barrier();

        // dg: the suffix sums of dgamma over the chunk, the gamma_C term and the
        // prefix sums of W (all before token t), as scans across the 16 lanes
        // of a row: lane (t = tid % 16) of row j of wave w holds token t of
        // channels 16 w + 4 j .. + 3 (lanes past the row's end read 0).  And
        // this slice's share of dbeta.
        {
            const int t = tid & 15, c0 = 16 * w + 4 * ((tid >> 4) & 3);
            f32x4 x = *reinterpret_cast<const f32x4 *>(&sDgam[t][c0]);
            const f32x4 ww = *reinterpret_cast<const f32x4 *>(&sW[t][c0]);
            f32x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = dpp_mv<0x111>(ww[i]);  // row_shr:1: W of token t - 1
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += dpp_mv<0x101>(x[i]);  // row_shl:1
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] += dpp_mv<0x111>(y[i]);  // row_shr:1
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += dpp_mv<0x102>(x[i]);  // row_shl:2
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] += dpp_mv<0x112>(y[i]);  // row_shr:2
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += dpp_mv<0x104>(x[i]);  // row_shl:4
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] += dpp_mv<0x114>(y[i]);  // row_shr:4
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] += dpp_mv<0x108>(x[i]);  // row_shl:8
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] += dpp_mv<0x118>(y[i]);  // row_shr:8
            f32x4 dg;
#pragma unroll
            for (int i = 0; i < 4; ++i) dg[i] = (x[i] + sDgC[c0 + i]) + y[i];
            st16(pg, 4 * (static_cast<uint32_t>(t) * HD + c0), dg);
            if (tid < kC) st4(pb, 4 * (static_cast<uint32_t>(tid) * static_cast<uint32_t>(H)), sDB[tid]);
        }
    }

    if (a.dh0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a.dh0[sb + (16 * w + 4 * g4 + i) * D + col0 + 16 * ct + r16] = dS[ct][i];
        }
    }
}

// A slice's partials are three planes of n_tok * D values (dq, dk, dg), then
// n_tok values (dbeta); slices start `stride` floats apart (a multiple of 4,
// so every plane of every slice starts 16-byte aligned).  The planes are
// summed four values at a time when dq, dk and dg are 16-byte aligned too
// (a plane holds a multiple of 16 values, so a group never straddles two).
template <bool VEC>
__global__ __launch_bounds__(256) void bwd_sum_kernel(const float *part, int64_t stride, int64_t plane, int ns,
                                                      float *dq, float *dk, float *dg, float *dbeta, int64_t n_tok) {
    constexpr int W = VEC ? 4 : 1;
    using V = std::conditional_t<VEC, f32x4, float>;
    const int64_t n_vec = 3 * plane / W, step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; e < n_vec + n_tok; e += step) {
        if (e < n_vec) {
            V s = *reinterpret_cast<const V *>(part + W * e);
            for (int sl = 1; sl < ns; ++sl) s += *reinterpret_cast<const V *>(part + sl * stride + W * e);
            const int64_t x = W * e;
            float *dst = x < plane ? dq + x : x < 2 * plane ? dk + (x - plane) : dg + (x - 2 * plane);
            __builtin_nontemporal_store(s, reinterpret_cast<V *>(dst));
        } else {
            const int64_t t = e - n_vec;
            float s = part[3 * plane + t];
            for (int sl = 1; sl < ns; ++sl) s += part[sl * stride + 3 * plane + t];
            dbeta[t] = s;
        }
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
    const int64_t BH = a.B * a.H;
    if (a.D == 128) {
        // bf16 inputs: the chunk form on the matrix cores.  fp32 inputs: the
        // token-serial adjoint, whose dg is formed per token; in the chunk
        // form dg sums pieces that partly cancel, which costs it about 1e-4
        // of accuracy (relative to its rms) under strong decay or beta = 1.
        // (the chunk kernel's 32-bit byte offsets need 16 H D 4 < 2^31)
        const dim3 grid(static_cast<unsigned>(BH * 4));
        if (a.bf16 && a.H < 65536) hipLaunchKernelGGL(bwd_chunk_kernel, grid, dim3(512), 0, s, a);
        else if (a.bf16) hipLaunchKernelGGL((bwd_col_kernel<true>), grid, dim3(512), 0, s, a);
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
    const bool vec = ((reinterpret_cast<uintptr_t>(a.dq) | reinterpret_cast<uintptr_t>(a.dk) |
                       reinterpret_cast<uintptr_t>(a.dg)) & 15) == 0;
    const int64_t total = 3 * a.part_plane / (vec ? 4 : 1) + n_tok;
    const int64_t blocks = (total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192;
    const int ns = a.D == 128 ? 4 : 1;
    if (blocks > 0 && vec)
        hipLaunchKernelGGL(bwd_sum_kernel<true>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a.part,
                           a.part_stride, a.part_plane, ns, a.dq, a.dk, a.dg, a.dbeta, n_tok);
    else if (blocks > 0)
        hipLaunchKernelGGL(bwd_sum_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a.part,
                           a.part_stride, a.part_plane, ns, a.dq, a.dk, a.dg, a.dbeta, n_tok);
    return hipGetLastError();
}

}  // namespace kda
