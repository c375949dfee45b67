// kda_prefill_mfma.hip -- chunked KDA prefill on the gfx950 matrix cores.
//
// Handles bf16 q/k/v with d_k = d_v = 128 (fp32 gates, state and output).
// One work-group per (batch, head, 32-column value slice): 4 slices per head,
// so a 56-head sequence runs on 224 work-groups.  The slices of one head are
// placed on the same XCD (blockIdx -> XCD is round-robin), so their repeated
// reads of q, k, g hit that XCD's L2.
//
// Chunk form for a 16-token chunk with start state S0 (rows = key channels),
// per-channel cumulative log-decay gamma_r = g_1 + ... + g_r and
// gamma_C = gamma_16:
//   Qb = q * e^gamma      Kb = k * e^gamma      Kh = k * e^-gamma
//   Kd = k * e^(gamma_C - gamma)
//   A  = strict_lower(diag(beta) Kb Kh^T)        (I + A) is unit lower triangular
//   P  = lower(Qb Kh^T)
//   M  = (I + A)^-1 diag(beta)
//   X  = Kb S0,   Y = Qb S0                      (the two state contractions)
//   U  = M (V - X)
//   O  = scale * (Y + P U)
//   S  = diag(e^gamma_C) S0 + Kd^T U
// The 16-token chunk with gates >= -5 keeps every e^(+-gamma) inside the bf16
// normal range, so all products can use bf16 matrix instructions (Kimi K3
// paper digest, devpress.csdn.net, section 2.1 (1)).  Each product is taken
// in three bf16 passes (x = x_hi + x_lo; a*b ~ a_hi b_hi + a_hi b_lo +
// a_lo b_hi) with fp32 accumulation, which keeps fp32-level accuracy.
//
// Work split inside a work-group (4 waves): wave w owns key channels
// [32w, 32w + 32).  It computes the decay factors and scaled operands of those
// channels, their contributions to the 16x16 Gram matrices (A, P) and to X, Y,
// and holds the matching 32 rows of the state slice in registers.  Partial
// Grams and partial X, Y are summed across waves through LDS; wave 0 solves
// the triangular system.
//
// Operand layouts (v_mfma_f32_16x16x16bf16_1k / 16x16x32_bf16, lane l,
// group g = l / 16, n = l % 16):
//   16x16x16:  A[m = n][k = 4g + i],  B[k = 4g + i][col = n],  i < 4
//   16x16x32:  A[m = n][k = 8g + j],  B[k = 8g + j][col = n],  j < 8
//   result:    C[row = 4g + i][col = n]
// Key-channel data is produced in the "channel per lane" layout (channel n,
// tokens 4g..4g+3), which is directly the A operand of the contractions over
// tokens (Kd^T U).  A 16x16x16 product with the identity turns it into the
// "token per lane" layout (token n, channels 4g..4g+3) needed by the
// contractions over channels; the results are exact because the inputs are
// already bf16.  For the 16x16x32 channel contractions, slot j < 4 of group g
// is channel 4g + j of the wave's first 16-channel tile and slot j >= 4 is
// channel 4g + j - 4 of its second tile; the state rows are held in the same
// order (the result layout of two 16-row tiles), so both operands agree.
#include "kda_internal.h"

namespace kda {
namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));
using bf16x4 = __bf16 __attribute__((ext_vector_type(4)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using s16x4 = short __attribute__((ext_vector_type(4)));

constexpr int kD = 128;     // head dimension (d_k = d_v)
constexpr int kDVS = 32;    // value columns per work-group
constexpr int kNV = kD / kDVS;
constexpr int kC = kChunk;  // 16

__device__ __forceinline__ f32x4 mfma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Sp4 {
    bf16x4 hi, lo;
};
struct Sp8 {
    bf16x8 hi, lo;
};

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both round-to-nearest.
__device__ __forceinline__ Sp4 split4(f32x4 x) {
    Sp4 s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const __bf16 h = static_cast<__bf16>(x[i]);
        s.hi[i] = h;
        s.lo[i] = static_cast<__bf16>(x[i] - static_cast<float>(h));
    }
    return s;
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Sp8 cat8(Sp4 a, Sp4 b) { return Sp8{cat8(a.hi, b.hi), cat8(a.lo, b.lo)}; }

// Three-pass products: c + a * b with fp32-level accuracy.
// For K = 16 the three passes fit in two 16x16x32 products: slots 0-3 of a
// lane group carry one pass and slots 4-7 another, over the same 4 k.
// (Both products use the same opcode: a 16x16x16 product that accumulates
// onto a just-issued 16x16x32 result was observed to read a stale value.)
__device__ __forceinline__ f32x4 mm16(const Sp4 &a, const Sp4 &b, f32x4 c) {
    const bf16x4 z = {};
    c = mfma32(cat8(a.hi, a.lo), cat8(b.hi, b.hi), c);
    c = mfma32(cat8(a.hi, z), cat8(b.lo, z), c);
    return c;
}
__device__ __forceinline__ f32x4 mm32(const Sp8 &a, const Sp8 &b, f32x4 c) {
    c = mfma32(a.hi, b.hi, c);
    c = mfma32(a.hi, b.lo, c);
    c = mfma32(a.lo, b.hi, c);
    return c;
}

// bf16 values (exact) from an fp32 result vector.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}

// "channel per lane" -> "token per lane" for one 16x16 bf16 tile, exact.
__device__ __forceinline__ bf16x4 transpose_tile(bf16x4 x, bf16x4 ident) {
    return to_bf16x4(mfma16(x, ident, f32x4{0.f, 0.f, 0.f, 0.f}));
}

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// One chunk's raw inputs for one lane: g, q, k of the wave's two channel tiles
// ("channel per lane": channel 16*(2w+tt) + n16, tokens 4g + i), v of the two
// value-column tiles (token 4g + i, column 16c + n16), and beta of token tid.
struct RawChunk {
    float g[2][4];
    uint16_t q[2][4], k[2][4], v[2][4];
    float beta;
};

__device__ __forceinline__ void load_raw(RawChunk &r, const PrefillArgs &a, int64_t t0, int64_t b, int64_t h, int w,
                                         int grp, int n16, int col0, int tid) {
    const uint16_t *q = static_cast<const uint16_t *>(a.q);
    const uint16_t *k = static_cast<const uint16_t *>(a.k);
    const uint16_t *v = static_cast<const uint16_t *>(a.v);
    const int64_t T = a.T, H = a.H, last = T - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t t = min(t0 + 4 * grp + i, last);
        const int64_t row = ((b * T + t) * H + h) * kD;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int64_t idx = row + 16 * (2 * w + tt) + n16;
            r.g[tt][i] = a.g[idx];
            r.q[tt][i] = q[idx];
            r.k[tt][i] = k[idx];
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) r.v[c][i] = v[row + col0 + 16 * c + n16];
    }
    r.beta = (tid < kC) ? a.beta[(b * T + min(t0 + tid, last)) * H + h] : 0.f;
}

template <typename InT>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
    __shared__ float sGram[4][2][kC][kC];      // per-wave partial Grams: [wave][A/P][r][s]
    __shared__ float sXY[4][2][2][kC][kC];     // per-wave partial X, Y: [wave][X/Y][col tile][r][col]
    __shared__ __attribute__((aligned(16))) float sA[kC][kC];  // summed A (with beta), read by the solver lanes
    __shared__ float sM[kC][kC + 1];           // M = (I + A)^-1 diag(beta)
    __shared__ float sP[kC][kC + 1];           // P (lower triangle incl. diagonal)
    __shared__ float sEC[kD];                  // e^gamma_C per key channel
    __shared__ float sBeta[kC];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int grp = lane >> 4;
    const int n16 = lane & 15;

    // XCD-aware block mapping: block id -> (xcd = id % 8, k = id / 8); the 4
    // slices of head bh = (k / 4) * 8 + xcd run on the same XCD.
    const int64_t BH = a.B * a.H;
    const int64_t bid = blockIdx.x;
    const int64_t kk = bid >> 3;
    const int64_t bh = (kk >> 2) * 8 + (bid & 7);
    const int nv = static_cast<int>(kk & 3);
    if (bh >= BH) return;  // padding blocks of the last XCD round
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t T = a.T, H = a.H;
    const int col0 = nv * kDVS;

    // identity operand for the layout transposes: B[k = 4g + i][col = n] = (4g + i == n)
    bf16x4 ident;
#pragma unroll
    for (int i = 0; i < 4; ++i) ident[i] = static_cast<__bf16>((4 * grp + i == n16) ? 1.f : 0.f);

    // State slice rows 16*(2w+tt) + 4*grp + i, columns col0 + 16*c + n16.
    f32x4 Sacc[2][2];
    const int64_t sbase = bh * kD * kD;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (2 * w + tt) + 4 * grp + i;
                Sacc[tt][c][i] = a.h0 ? a.h0[sbase + row * kD + col0 + 16 * c + n16] : 0.f;
            }
        }
    }

    const int64_t nchunks = (T + kC - 1) / kC;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // Raw inputs of one chunk for this lane.  Loads use a clamped token index
    // so they never branch or leave the sequence; tokens past T are masked to
    // identity steps (g = 0, q = k = v = 0, beta = 0) when the chunk is used.
    // The next chunk's loads are issued before the current chunk is computed.
    RawChunk nxt;
    if (nchunks > 0) load_raw(nxt, a, 0, b, h, w, grp, n16, col0, tid);

    for (int64_t n = 0; n < nchunks; ++n) {
        const int64_t t0 = n * kC;
        const RawChunk cur = nxt;
        if (n + 1 < nchunks) load_raw(nxt, a, t0 + kC, b, h, w, grp, n16, col0, tid);
        bool valid[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) valid[i] = t0 + 4 * grp + i < T;

        // ---- decay factors and scaled operands, "channel per lane" layout ----
        Sp4 Qb[2], Kb[2], Kh[2], Kd[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int ch = 16 * (2 * w + tt) + n16;
            float gv[4], qv[4], kv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                gv[i] = valid[i] ? cur.g[tt][i] : 0.f;
                qv[i] = valid[i] ? bf16_bits_to_float(cur.q[tt][i]) : 0.f;
                kv[i] = valid[i] ? bf16_bits_to_float(cur.k[tt][i]) : 0.f;
            }
            // prefix sums of the log-decay: in-lane over 4 tokens, then across
            // the 4 token groups of the channel (lanes n16 + 16 g')
            float cum[4];
            cum[0] = gv[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) cum[i] = cum[i - 1] + gv[i];
            const float s0 = __shfl(cum[3], n16);
            const float s1 = __shfl(cum[3], n16 + 16);
            const float s2 = __shfl(cum[3], n16 + 32);
            const float s3 = __shfl(cum[3], n16 + 48);
            const float before = ((grp >= 1 ? s0 : 0.f) + (grp >= 2 ? s1 : 0.f)) + (grp >= 3 ? s2 : 0.f);
            const float gC = ((s0 + s1) + s2) + s3;
            f32x4 qb, kb, kh, kd;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float gam = before + cum[i];
                const float ep = __expf(gam);
                const float em = __expf(-gam);
                const float ed = __expf(gC - gam);
                qb[i] = qv[i] * ep;
                kb[i] = kv[i] * ep;
                kh[i] = kv[i] * em;
                kd[i] = kv[i] * ed;
            }
            Qb[tt] = split4(qb);
            Kb[tt] = split4(kb);
            Kh[tt] = split4(kh);
            Kd[tt] = split4(kd);
            if (grp == 0) sEC[ch] = __expf(gC);
        }
        if (tid < kC) sBeta[tid] = (t0 + tid < T) ? cur.beta : 0.f;

        // ---- "token per lane" operands for the contractions over channels ----
        Sp8 QbT, KbT, KhT;
        QbT.hi = cat8(transpose_tile(Qb[0].hi, ident), transpose_tile(Qb[1].hi, ident));
        QbT.lo = cat8(transpose_tile(Qb[0].lo, ident), transpose_tile(Qb[1].lo, ident));
        KbT.hi = cat8(transpose_tile(Kb[0].hi, ident), transpose_tile(Kb[1].hi, ident));
        KbT.lo = cat8(transpose_tile(Kb[0].lo, ident), transpose_tile(Kb[1].lo, ident));
        KhT.hi = cat8(transpose_tile(Kh[0].hi, ident), transpose_tile(Kh[1].hi, ident));
        KhT.lo = cat8(transpose_tile(Kh[0].lo, ident), transpose_tile(Kh[1].lo, ident));

        // ---- partial Grams over this wave's 32 channels ----
        const f32x4 Aw = mm32(KbT, KhT, zero);
        const f32x4 Pw = mm32(QbT, KhT, zero);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sGram[w][0][4 * grp + i][n16] = Aw[i];
            sGram[w][1][4 * grp + i][n16] = Pw[i];
        }

        // ---- partial X = Kb S0 and Y = Qb S0 over this wave's channels ----
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const Sp8 Sb = cat8(split4(Sacc[0][c]), split4(Sacc[1][c]));
            const f32x4 Xw = mm32(KbT, Sb, zero);
            const f32x4 Yw = mm32(QbT, Sb, zero);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sXY[w][0][c][4 * grp + i][n16] = Xw[i];
                sXY[w][1][c][4 * grp + i][n16] = Yw[i];
            }
        }
        __syncthreads();  // (1) partial Grams and X, Y are in LDS

        // ---- wave 0: (I + A) M = diag(beta) by forward substitution ----
        if (w == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = (lane * 4 + e) >> 4, s = (lane * 4 + e) & 15;
                const float as = sGram[0][0][r][s] + sGram[1][0][r][s] + sGram[2][0][r][s] + sGram[3][0][r][s];
                const float ps = sGram[0][1][r][s] + sGram[1][1][r][s] + sGram[2][1][r][s] + sGram[3][1][r][s];
                sA[r][s] = (s < r) ? sBeta[r] * as : 0.f;
                sP[r][s] = (s <= r) ? ps : 0.f;
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            if (lane < kC) {
                const int s = lane;
                float Ar[kC][kC];
#pragma unroll
                for (int r = 0; r < kC; ++r) {
#pragma unroll
                    for (int u4 = 0; u4 < kC / 4; ++u4) {
                        const f32x4 row = *reinterpret_cast<const f32x4 *>(&sA[r][4 * u4]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) Ar[r][4 * u4 + j] = row[j];
                    }
                }
                // right-looking substitution: independent updates per pivot
                float x[kC];
#pragma unroll
                for (int r = 0; r < kC; ++r) x[r] = (r == s) ? 1.f : 0.f;
#pragma unroll
                for (int u = 0; u < kC - 1; ++u) {
#pragma unroll
                    for (int r = u + 1; r < kC; ++r) x[r] -= Ar[r][u] * x[u];
                }
                const float bs = sBeta[s];
#pragma unroll
                for (int r = 0; r < kC; ++r) sM[r][s] = x[r] * bs;
            }
        }

        // ---- every wave: Z = V - X for both column tiles (sum of partials) ----
        Sp4 Z[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4 zc;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * grp + i;
                const float vv = valid[i] ? bf16_bits_to_float(cur.v[c][i]) : 0.f;
                const float xs = sXY[0][0][c][r][n16] + sXY[1][0][c][r][n16] + sXY[2][0][c][r][n16] + sXY[3][0][c][r][n16];
                zc[i] = vv - xs;
            }
            Z[c] = split4(zc);
        }
        f32x4 Yred = zero;
        if (w < 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * grp + i;
                Yred[i] = sXY[0][1][w][r][n16] + sXY[1][1][w][r][n16] + sXY[2][1][w][r][n16] + sXY[3][1][w][r][n16];
            }
        }
        float eCrow[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) eCrow[tt][i] = sEC[16 * (2 * w + tt) + 4 * grp + i];
        }
        __syncthreads();  // (2) M and P are in LDS

        // ---- U = M Z ----
        f32x4 mfrag, pfrag;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            mfrag[i] = sM[n16][4 * grp + i];
            pfrag[i] = sP[n16][4 * grp + i];
        }
        const Sp4 Mf = split4(mfrag);
        Sp4 Uc[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) Uc[c] = split4(mm16(Mf, Z[c], zero));

        // ---- O = scale * (Y + P U), waves 0 and 1 write column tiles 0 and 1 ----
        if (w < 2) {
            const Sp4 Pf = split4(pfrag);
            Sp4 Uw;  // select without a run-time register-array index (which would go to scratch)
            Uw.hi = (w == 0) ? Uc[0].hi : Uc[1].hi;
            Uw.lo = (w == 0) ? Uc[0].lo : Uc[1].lo;
            const f32x4 O = mm16(Pf, Uw, Yred);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t t = t0 + 4 * grp + i;
                if (valid[i]) a.o[((b * T + t) * H + h) * kD + col0 + 16 * w + n16] = a.scale * O[i];
            }
        }

        // ---- S = diag(e^gamma_C) S0 + Kd^T U ----
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                f32x4 s0;
#pragma unroll
                for (int i = 0; i < 4; ++i) s0[i] = eCrow[tt][i] * Sacc[tt][c][i];
                Sacc[tt][c] = mm16(Kd[tt], Uc[c], s0);
            }
        }
        // Every LDS read of this chunk precedes barrier (2) except the M and P
        // fragments; this barrier keeps the next chunk's LDS writes behind them.
        __syncthreads();
    }

    if (a.hT) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * (2 * w + tt) + 4 * grp + i;
                    a.hT[sbase + row * kD + col0 + 16 * c + n16] = Sacc[tt][c][i];
                }
            }
        }
    }
}

}  // namespace

bool prefill_mfma_supported(const PrefillArgs &a) {
    if (a.D != kD || !a.bf16) return false;
    const char *env = getenv("KDA_DISABLE_MFMA");
    return !(env && env[0] == '1');
}

hipError_t launch_prefill_mfma(const PrefillArgs &a, hipStream_t s) {
    const int64_t BH = a.B * a.H;
    const int64_t rounds = (BH + 7) / 8;
    dim3 grid(static_cast<unsigned>(rounds * 8 * kNV)), block(256);
    hipLaunchKernelGGL(prefill_mfma_kernel<uint16_t>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
