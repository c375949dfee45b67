// kda_prefill_f32.hip -- chunked KDA prefill for fp32 q, k, v at d = 128 on the
// fp32 matrix cores (16x16x4 products, fp32 operands and accumulation).
//
// The 16-token chunk form ("Kimi K3 Architecture Explained", section 3, and
// the Kimi K3 paper digest, devpress.csdn.net, section 2.1 (1) for the chunk
// length): with start state S0, per-channel cumulative log-decay gamma and
// D_C = diag(e^gamma_C),
//   Qb = q e^gamma, Kb = k e^gamma, Kh = k e^-gamma
//   A = strict_lower(diag(beta) Kb Kh^T),  M = (I + A)^-1 diag(beta)
//   P = lower(Qb Kh^T),  Z = V - Kb S0,  U = M Z
//   O = scale (Qb S0 + P U),  S = D_C (S0 + Kh^T U)
// which regroups the token recurrence exactly.  Every product is an fp32
// 16 x 16 output tile with operands read from LDS, so the results carry fp32
// rounding only (the bf16 kernel splits its operands into bf16 pairs instead).
//
// One work-group per (b, h, 32-column slice), eight waves; waves w and w + 4
// share a SIMD.  Wave w holds rows 16 w .. 16 w + 15 of the slice's state in
// registers (both 16-column tiles).  A chunk runs in five phases with four
// work-group barriers that order LDS only:
//   L   the inputs to LDS, the decay factors and scaled operands formed on
//       the way (gamma summed in token order across a 16-lane row);
//   F1  Kb Kh^T -> A (wave 0), Qb Kh^T -> P (wave 1), Z = V - Kb S0 (waves 2,
//       3, one column tile each), and Qb S0 in channel halves (waves 4 .. 7);
//   F2  the solve for M (waves 0 .. 3, four columns each), while every wave
//       issues the next chunk's loads;
//   F3  U = M Z, then O = P U + scale Qb S0 from U's registers (waves 0, 1);
//   F4  every wave updates its state tiles and writes them to LDS for the
//       next chunk's products.
// L writes a second set of buffers on alternate chunks, so the next chunk's
// L needs no barrier after F4.
#include "kda_f32mfma.h"

namespace kda {
namespace {

constexpr int kF32D = 128, kF32CW = 32, kF32C = 16;

// The inputs of one chunk for thread tid (wave w, lane l): token l % 16,
// channels 16 w + 4 (l / 16) .. + 3 of q, k and g; the value slice's token
// (tid % 128) / 8, columns 4 (tid % 8) ..; beta of token tid % 16.
struct F32In {
    float4 q, k, g, v;
    float beta;
};

__device__ __forceinline__ F32In load_f32_inputs(const PrefillArgs &a, int64_t tok0, int nt, int col0, int tid) {
    constexpr int D = kF32D;
    const uint32_t H = static_cast<uint32_t>(a.H), HD = H * D, last = static_cast<uint32_t>(nt - 1) * HD;
    const uint32_t off = static_cast<uint32_t>(tid & 15) * HD + 16 * (tid >> 6) + 4 * ((tid >> 4) & 3);  // elements
    const Rsrc rq = buf(static_cast<const float *>(a.q) + tok0 * D, 4 * (last + D));
    const Rsrc rk = buf(static_cast<const float *>(a.k) + tok0 * D, 4 * (last + D));
    const Rsrc rg = buf(static_cast<const float *>(a.g) + tok0 * D, 4 * (last + D));
    const Rsrc rv = a.v ? buf(static_cast<const float *>(a.v) + tok0 * D + col0, 4 * (last + kF32CW)) : buf(nullptr, 0);
    const Rsrc rb = buf(a.beta + tok0, 4 * (static_cast<uint32_t>(nt - 1) * H + 1));
    F32In in;
    in.q = ld16f(rq, 4 * off);
    in.k = ld16f(rk, 4 * off);
    in.g = ld16f(rg, 4 * off);
    const int l = tid & 127;
    in.v = ld16f(rv, 4 * (static_cast<uint32_t>(l >> 3) * HD + 4 * (l & 7)));
    in.beta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, 4 * (static_cast<uint32_t>(tid & 15) * H), 0, 0));
    return in;
}

// e^x as 2^(x log2 e) on the hardware exp2, with the rounding of the product
// carried separately: x log2 e = yh + yl, where yh is the fp32 product, fma
// gives its exact residual and x (log2 e - c) adds the error of the constant
// c; then 2^(yh + yl) = 2^yh (1 + yl ln 2) to within yl^2, which is below
// 2^-40 here (|x| <= 80 + 16 at the floor gate).  Six operations, and the
// error of the hardware exp2 instead of |x| 2^-24.
__device__ __forceinline__ float exp_split(float x) {
    constexpr float kC = 1.44269502162933349609375f;  // log2 e, rounded to fp32
    constexpr float kCLo = 1.925963001e-8f;           // log2 e - kC
    constexpr float kLn2 = 0.693147182464599609375f;  // ln 2, rounded to fp32
    const float yh = x * kC;
    const float yl = __builtin_fmaf(x, kC, -yh) + x * kCLo;
    return __builtin_amdgcn_exp2f(yh) * __builtin_fmaf(yl, kLn2, 1.f);
}

template <int P, int PS>
struct F32Buf {
    float Qb[kF32C][P], Kb[kF32C][P], Kh[kF32C][P];
    float V[kF32C][PS];
    float egc[kF32D];  // e^gamma_C
    float beta[kF32C];
};

// (L) the chunk's operands.  Tokens past the end were loaded as zeros; their
// gate is set to 0 (a logit of 0 is not a zero gate), so they keep the last
// token's gamma and, with beta = 0 and zero q, k and v, change nothing.
template <int P, int PS>
__device__ __forceinline__ void store_f32_inputs(const PrefillArgs &a, const F32In &in, int nt, int tid,
                                                 F32Buf<P, PS> &bf) {
    const int t = tid & 15, c0 = 16 * (tid >> 6) + 4 * ((tid >> 4) & 3);
    float g0[4] = {in.g.x, in.g.y, in.g.z, in.g.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (a.gate == kGateLogitF32) g0[j] = gate_of_logit(g0[j], a.g_min);
        g0[j] = t < nt ? g0[j] : 0.f;
    }
    // gamma in token order: fifteen rounds of "the previous lane's sum plus my
    // g" leave lane t with ((g_0 + g_1) + ...) + g_t (the lane before the row's
    // start reads 0)
    float gam[4] = {g0[0], g0[1], g0[2], g0[3]};
#pragma unroll
    for (int st = 1; st < 16; ++st) {
#pragma unroll
        for (int j = 0; j < 4; ++j) gam[j] = dpp_mv<0x111>(gam[j]) + g0[j];  // row_shr:1
    }
    const float qv[4] = {in.q.x, in.q.y, in.q.z, in.q.w}, kv[4] = {in.k.x, in.k.y, in.k.z, in.k.w};
    f32x4 qb, kb, kh, eg;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float e = exp_split(gam[j]), ei = exp_split(-gam[j]);
        qb[j] = qv[j] * e;
        kb[j] = kv[j] * e;
        kh[j] = kv[j] * ei;
        eg[j] = e;
    }
    *reinterpret_cast<f32x4 *>(&bf.Qb[t][c0]) = qb;
    *reinterpret_cast<f32x4 *>(&bf.Kb[t][c0]) = kb;
    *reinterpret_cast<f32x4 *>(&bf.Kh[t][c0]) = kh;
    if (t == kF32C - 1) *reinterpret_cast<f32x4 *>(&bf.egc[c0]) = eg;
    if (tid < 128) *reinterpret_cast<f32x4 *>(&bf.V[tid >> 3][4 * (tid & 7)]) = f32x4{in.v.x, in.v.y, in.v.z, in.v.w};
    if (tid < kF32C) bf.beta[tid] = in.beta;
}

__global__ __launch_bounds__(512) void prefill_f32_kernel(PrefillArgs a) {
    constexpr int D = kF32D, kCW = kF32CW, kNS = D / kCW, kC = kF32C;
    constexpr int kP = 132;   // pitch of the token x channel arrays
    constexpr int kPS = 36;   // pitch of the token x column arrays
    constexpr int kP16 = 20;  // pitch of the 16 x 16 arrays
    __shared__ F32Buf<kP, kPS> sIn[2];             // L's buffers, by chunk parity
    __shared__ float sS0T[kCW][kP];                // the chunk's start state, transposed: column j, channel c
    __shared__ float sZ[kC][kPS], sU[kC][kPS], sY[2][kC][kPS];
    __shared__ float sA[kC][kP16], sPs[kC][kP16], sM[kC][kP16];

    const int64_t bh = blockIdx.x / kNS;
    const int slice = static_cast<int>(blockIdx.x % kNS);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int tid_k = threadIdx.x, lane0 = tid_k & 63, r16_0 = lane0 & 15, g4_0 = lane0 >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid_k >> 6);  // wave-uniform
    const int64_t T = a.T, H = a.H;
    const int col0 = slice * kCW;
    const int64_t sb = bh * D * D;
    const uint32_t HD = static_cast<uint32_t>(a.H) * D;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    // this wave's state tiles: tile ct is rows 16 w .., columns 16 ct .. of
    // the slice; component i is row 4 g4 + i of the block
    f32x4 S[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[ct][i] = a.h0 ? a.h0[sb + (16 * w + 4 * g4_0 + i) * D + col0 + 16 * ct + r16_0] : 0.f;
        *reinterpret_cast<f32x4 *>(&sS0T[16 * ct + r16_0][16 * w + 4 * g4_0]) = S[ct];
    }

    const int64_t nch = (T + kC - 1) / kC;
    F32In in{};
    if (nch > 0) in = load_f32_inputs(a, (b * T) * H + h, static_cast<int>(T < kC ? T : kC), col0, tid_k);
    int64_t ck_left = a.ckpt_every, ck_i = 0;  // chunks to the next checkpoint, its index
    for (int64_t n = 0; n < nch; ++n) {
        const int64_t t0 = n * kC;
        const int nt = static_cast<int>(t0 + kC < T ? kC : T - t0);
        const int par = static_cast<int>(n & 1);
        // the lane's indices, made opaque once per chunk (LDS addresses are then
        // formed from a few registers rather than kept across the loop)
        int tidv = tid_k;
        asm volatile("" : "+v"(tidv));
        const int tid = tidv, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
        F32Buf<kP, kPS> &bf = sIn[par];
        const int64_t tok0 = (b * T + t0) * H + h;
        const uint32_t last = static_cast<uint32_t>(nt - 1) * HD;

        // (L)
        store_f32_inputs(a, in, nt, tid, bf);
        lds_barrier();

        // (F1)
        if (w == 0) {
            const f32x4 gr = tile_mm_kc<D>(&bf.Kb[0][0], kP, &bf.Kh[0][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                sA[r][r16] = r16 < r ? bf.beta[r] * gr[i] : 0.f;
            }
        } else if (w == 1) {
            const f32x4 pr = tile_mm_kc<D>(&bf.Qb[0][0], kP, &bf.Kh[0][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                sPs[r][r16] = r16 <= r ? a.scale * pr[i] : 0.f;
            }
        } else if (w < 4) {
            const int ct = w - 2;
            const f32x4 x = tile_mm_kc<D>(&bf.Kb[0][0], kP, &sS0T[16 * ct][0], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g4 + i;
                sZ[t][16 * ct + r16] = bf.V[t][16 * ct + r16] - x[i];
            }
        } else {
            const int ct = (w - 4) & 1, kh = (w - 4) >> 1;
            const f32x4 y = tile_mm_kc<64>(&bf.Qb[0][64 * kh], kP, &sS0T[16 * ct][64 * kh], kP, zero, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) sY[kh][4 * g4 + i][16 * ct + r16] = y[i];
        }
        lds_barrier();

        // (F2) M = (I + A)^-1 diag(beta): row group g4 of wave w < 4 solves
        // column 4 w + g4.  Every wave first issues the next chunk's loads (in
        // the last step, this chunk's again: the loads are the same every step).
        {
            const int64_t nn = n + 1 < nch ? n + 1 : n;
            const int64_t tn = nn * kC;
            in = load_f32_inputs(a, (b * T + tn) * H + h, static_cast<int>(tn + kC < T ? kC : T - tn), col0, tid);
        }
        if (w < 4) {
            float nar[kC];
#pragma unroll
            for (int u = 0; u < kC; ++u) nar[u] = -sA[r16][u];
            const int s = 4 * w + g4;
            float x = r16 == s ? 1.f : 0.f;
            solve_pivots<0>(x, nar);
            sM[r16][s] = x * bf.beta[s];
        }
        lds_barrier();

        // (F3) U = M Z, then O = P U + scale Qb S0 (waves 0, 1: column tile w).
        // U's result is O's operand from registers: lane (r16, g4) holds rows
        // 4 g4 + i of U's column r16, its values when the product takes
        // k = 4 g4 + m at step m.
        if (w < 2) {
            const int ct = w;
            const f32x4 u = tile_mm<kC>(&sM[0][0], kP16, 1, &sZ[0][16 * ct], kPS, 1, zero, lane);
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 4 * g4 + i;
                sU[t][16 * ct + r16] = u[i];
                o[i] = a.scale * (sY[0][t][16 * ct + r16] + sY[1][t][16 * ct + r16]);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) o = mfma4(sPs[r16][4 * g4 + m], u[m], o);
            if (a.o) {
                const Rsrc ro = buf(a.o + tok0 * D + col0, 4 * (last + kCW));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    st4(ro, 4 * (static_cast<uint32_t>(4 * g4 + i) * HD + 16 * ct + r16), o[i]);
            }
        }
        lds_barrier();

        // (F4) S = D_C (S0 + Kh^T U) on this wave's tiles, then the transposed
        // copy for the next chunk's products (F1 reads it after the next L's
        // barrier; this chunk's F1 read it before F1's)
        {
            const f32x4 egc = *reinterpret_cast<const f32x4 *>(&bf.egc[16 * w + 4 * g4]);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const f32x4 upd = tile_mm<kC>(&bf.Kh[0][16 * w], 1, kP, &sU[0][16 * ct], kPS, 1, zero, lane);
                S[ct] = egc * (S[ct] + upd);
                *reinterpret_cast<f32x4 *>(&sS0T[16 * ct + r16][16 * w + 4 * g4]) = S[ct];
            }
        }
        if (a.ckpt && --ck_left == 0) {  // the state after (ck_i + 1) * ckpt_every chunks
            if (ck_i < a.n_ckpt) {
                float *ck = a.ckpt + ck_i * (a.B * H * D * D) + sb;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) ck[(16 * w + 4 * g4 + i) * D + col0 + 16 * ct + r16] = S[ct][i];
            }
            ++ck_i;
            ck_left = a.ckpt_every;
        }
    }

    if (a.hT) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) a.hT[sb + (16 * w + 4 * g4_0 + i) * D + col0 + 16 * ct + r16_0] = S[ct][i];
    }
}

}  // namespace

bool prefill_f32_supported(const PrefillArgs &a) {
    // fp32 q, k, v at d = 128 with an fp32 gate (log-decay or logits), without
    // the q/k normalisation; the kernel's 32-bit in-chunk byte offsets need
    // 16 H 128 4 < 2^31, i.e. H < 65536
    return !a.bf16 && a.D == kF32D && a.H < 65536 && !a.qk_norm &&
           (a.gate == kGateLogDecay || a.gate == kGateLogitF32);
}

hipError_t launch_prefill_f32(const PrefillArgs &a, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(a.B * a.H * (kF32D / kF32CW)));
    hipLaunchKernelGGL(prefill_f32_kernel, grid, dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
