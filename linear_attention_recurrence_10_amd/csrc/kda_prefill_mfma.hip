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
// [32w, 32w + 32) = 16-channel tiles 2w and 2w + 1.  It loads and scales
// those channels, forms their contributions to the 16x16 Gram matrices and to
// X, Y, and holds the matching 32 rows of the state slice in registers.
// Partial Grams and partial X, Y are summed across waves through LDS; wave 0
// solves the triangular system.
//
// Operand layouts (lane l, row group g = l / 16, n = l % 16):
//   16x16x16 (bf16_1k):  A[m = n][k = 4g + i],  B[k = 4g + i][col = n]
//   16x16x32 (bf16):     A[m = n][k = 8g + j],  B[k = 8g + j][col = n]
//   result:              C[row = 4g + i][col = n]
// "Token per lane": lane (n, g) holds token n of the chunk and, in slot j of
// an 8-wide operand, key channel 16 (2w) + 4g + j (j < 4) or
// 16 (2w + 1) + 4g + j - 4 (j >= 4).  This is the operand layout of every
// contraction over channels (X, Y, the Grams); the state rows are kept in the
// result layout of two 16-row tiles, which lists the same channels in the
// same slots.  q, k, g are loaded straight into it with 8- and 16-byte loads,
// and the cumulative decay over tokens is a prefix sum across the 16 lanes of
// a row (DPP row shifts).  Kd, the operand of the contraction over tokens,
// needs "channel per lane" (channel n, tokens 4g .. 4g + 3): a 16x16x16
// product with the identity converts it exactly (its inputs are bf16).  The
// Grams are formed transposed (Kh Kb^T, Kh Qb^T), so their result layout is
// "row n, columns 4g + i", the A-operand layout of U = M Z and P U.
#include <type_traits>

#include "kda_internal.h"

namespace kda {
namespace {

using f32x4 = float __attribute__((ext_vector_type(4)));
using bf16x4 = __bf16 __attribute__((ext_vector_type(4)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using s16x4 = short __attribute__((ext_vector_type(4)));
using u32x2 = uint32_t __attribute__((ext_vector_type(2)));
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
using f32x2 = float __attribute__((ext_vector_type(2)));
using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));

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

// x = hi + lo with hi = x truncated to bf16 (its upper 16 bits, so x - hi is
// exact) and lo = bf16(x - hi) rounded to nearest: |x - hi - lo| <= 2^-16 |x|.
// Per pair of values: one byte permute packs the two hi halves, one
// conversion packs the two lo values.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    const uint32_t u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
    hi = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // [upper half of u0, upper half of u1]
    const float l0 = x0 - __uint_as_float(u0 & 0xffff0000u);
    const float l1 = x1 - __uint_as_float(u1 & 0xffff0000u);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){l0, l1}, bf16x2));
}
__device__ __forceinline__ Sp4 split4(f32x4 x) {
    uint32_t h0, h1, l0, l1;
    split_pair(x[0], x[1], h0, l0);
    split_pair(x[2], x[3], h1, l1);
    return Sp4{__builtin_bit_cast(bf16x4, u32x2{h0, h1}), __builtin_bit_cast(bf16x4, u32x2{l0, l1})};
}
__device__ __forceinline__ Sp8 split8(const float (&x)[8]) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) split_pair(x[2 * p], x[2 * p + 1], h[p], l[p]);
    return Sp8{__builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]}),
               __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]})};
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ Sp8 cat8(Sp4 a, Sp4 b) { return Sp8{cat8(a.hi, b.hi), cat8(a.lo, b.lo)}; }
__device__ __forceinline__ bf16x4 first4(bf16x8 x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 last4(bf16x8 x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

// Three-pass products: c + a * b with fp32-level accuracy.
__device__ __forceinline__ f32x4 mm32(const Sp8 &a, const Sp8 &b, f32x4 c) {
    c = mfma32(a.hi, b.hi, c);
    c = mfma32(a.hi, b.lo, c);
    c = mfma32(a.lo, b.hi, c);
    return c;
}
// K = 16: three 16x16x16 products on the existing operand registers (no
// repacking).  A dependent chain keeps one opcode: a 16x16x16 product that
// accumulates onto a just-issued 16x16x32 result was observed to read a stale
// value, so K = 16 and K = 32 products never share an accumulator chain.
__device__ __forceinline__ f32x4 mm16(const Sp4 &a, const Sp4 &b, f32x4 c) {
    c = mfma16(a.hi, b.hi, c);
    c = mfma16(a.hi, b.lo, c);
    c = mfma16(a.lo, b.hi, c);
    return c;
}

// bf16 values (exact) from an fp32 result vector.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = static_cast<__bf16>(x[i]);
    return r;
}

// "token per lane" -> "channel per lane" for one 16x16 bf16 tile, exact.
__device__ __forceinline__ bf16x4 transpose_tile(bf16x4 x, bf16x4 ident) {
    return to_bf16x4(mfma16(x, ident, f32x4{0.f, 0.f, 0.f, 0.f}));
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// DPP data movement inside each 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
template <int U>
__device__ __forceinline__ float row_bcast(float x) {  // lane U of the row to the whole row
    return dpp_move<0x150 + U>(x);
}
// Inclusive prefix sum over the 16 lanes of each row (lanes shifted in from
// outside the row read 0).
__device__ __forceinline__ float row_prefix_sum(float x) {
    x += dpp_move<0x111>(x);  // row_shr:1
    x += dpp_move<0x112>(x);  // row_shr:2
    x += dpp_move<0x114>(x);  // row_shr:4
    x += dpp_move<0x118>(x);  // row_shr:8
    return x;
}

// Right-looking forward substitution for one column of (I + A)^-1: lane
// (row r = n, group g) holds X[r][s] for one column s per 16-lane row.  At
// pivot u every row subtracts A[r][u] times row u; row u of the same column
// lives in lane u of the same 16-lane row, so a DPP broadcast replaces any LDS
// traffic.  A is strictly lower triangular, so rows r <= u are unaffected
// (A[r][u] = 0).
template <int U>
__device__ __forceinline__ void tri_pivots(float &x, const float (&ar)[kC]) {
    if constexpr (U < kC - 1) {
        x = __builtin_fmaf(-ar[U], row_bcast<U>(x), x);
        tri_pivots<U + 1>(x, ar);
    }
}

// One chunk's raw inputs for one lane: q, k (4 bf16 per tile) and g (4 fp32
// per tile) of token n in the "token per lane" layout, beta of token n, and v
// in the result layout (token 4g + i, value column 16c + n of the slice).
struct RawChunk {
    u32x2 q[2], k[2];
    f32x4 g[2];
    uint16_t v[2][4];
    float beta;
};

// Loop-invariant element offsets of this lane's loads, relative to the first
// token row of the chunk for this (batch, head).
struct LaneOffsets {
    int tok[2];   // token n, channels 16 (2w + tt) + 4g .. + 3
    int v[2][4];  // token 4g + i, column col0 + 16c + n
};

__device__ __forceinline__ LaneOffsets lane_offsets(int64_t H, int w, int grp, int n16, int col0) {
    LaneOffsets o;
    const int HD = static_cast<int>(H) * kD;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) o.tok[tt] = n16 * HD + 16 * (2 * w + tt) + 4 * grp;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o.v[c][i] = (4 * grp + i) * HD + col0 + 16 * c + n16;
    }
    return o;
}

// Loads never branch per element and never leave the sequence: in a last,
// partial chunk the token index is clamped.  Offsets are unsigned 32-bit
// values added to a wave-uniform 64-bit base.
__device__ __forceinline__ void load_raw(RawChunk &r, const PrefillArgs &a, int64_t t0, int64_t b, int64_t h,
                                         const LaneOffsets &off, int grp, int n16) {
    const int64_t T = a.T, H = a.H;
    const int64_t row0 = (b * T + t0) * H + h;  // token row of the chunk start (wave uniform)
    const char *gb = reinterpret_cast<const char *>(a.g + row0 * kD);
    const char *qb = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.q) + row0 * kD);
    const char *kb = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k) + row0 * kD);
    const char *vb = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v) + row0 * kD);
    const char *betab = reinterpret_cast<const char *>(a.beta + row0);
    const int64_t rem = T - t0;
    const int HD = static_cast<int>(H) * kD;
    int tok_shift = 0, beta_tok = n16;
    int v_shift[4] = {0, 0, 0, 0};
    if (rem < kC) {
        const int last = static_cast<int>(rem) - 1;
        beta_tok = min(n16, last);
        tok_shift = (beta_tok - n16) * HD;
#pragma unroll
        for (int i = 0; i < 4; ++i) v_shift[i] = (min(4 * grp + i, last) - (4 * grp + i)) * HD;
    }
    // element offsets are < 2^31 / 4, so the byte offsets fit in 32 bits
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const uint32_t e = static_cast<uint32_t>(off.tok[tt] + tok_shift);
        r.q[tt] = *reinterpret_cast<const u32x2 *>(qb + 2u * e);
        r.k[tt] = *reinterpret_cast<const u32x2 *>(kb + 2u * e);
        r.g[tt] = *reinterpret_cast<const f32x4 *>(gb + 4u * e);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            r.v[c][i] = *reinterpret_cast<const uint16_t *>(vb + 2u * static_cast<uint32_t>(off.v[c][i] + v_shift[i]));
    }
    r.beta = *reinterpret_cast<const float *>(betab + 4u * static_cast<uint32_t>(beta_tok * static_cast<int>(H)));
}

// Shared memory, double-buffered by chunk parity: the k-side of chunk n + 1
// and the state part of chunk n run between the same two barriers.
struct Smem {
    f32x4 gram[2][4][2][kC][4];  // partial Grams [parity][wave][A/P][row][column group]
    f32x4 xy[2][4][2][2][kC][4];  // partial X, Y [parity][wave][X/Y][col tile][column][token group]
    f32x4 A[4][kC][4];            // per-wave copy of the summed A (beta applied, strict lower)
    float M[2][kC][kC];           // M = (I + A)^-1 diag(beta) [parity][row][column]
    float beta[2][kC];
};

// Everything of one chunk that depends only on its own inputs (not on the
// state), kept in registers from the iteration that computes it to the one
// that uses it.
struct KSide {
    Sp8 Qb, Kb;     // "token per lane" split operands of X = Kb S0 and Y = Qb S0
    Sp4 KdT[2];     // "channel per lane" split Kd of the state update, per tile
    float eC[8];    // e^gamma_C of the lane's 8 state rows
    f32x4 v[2];     // values, token 4g + i, column 16c + n (masked)
    float beta;     // beta of token n (masked)
};

// K-side of the chunk starting at t0: consumes the raw inputs in `raw`, then
// issues the next chunk's loads into the same registers (no register copy,
// so nothing waits on them), and leaves the partial Grams of this wave's
// channels in LDS.
// Tokens past the end of the sequence become identity steps: their gate is
// set to 0 and their beta to 0.  That zeroes their rows and columns of A and
// M, hence their rows of U, so their (finite) q, k and v never contribute.
__device__ __forceinline__ void kside(const PrefillArgs &a, Smem &sm, RawChunk &raw, int64_t t0, bool more,
                                      int64_t b, int64_t h, const LaneOffsets &off, int par, int w, int grp,
                                      int n16, const bf16x4 &ident, KSide &ks) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const bool tok_ok = t0 + n16 < a.T;
    float gv[8], qv[8], kv[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gv[4 * tt + i] = tok_ok ? raw.g[tt][i] : 0.f;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const uint32_t qp = raw.q[tt][p], kp = raw.k[tt][p];
            qv[4 * tt + 2 * p] = bf16_lo(qp);
            qv[4 * tt + 2 * p + 1] = bf16_hi(qp);
            kv[4 * tt + 2 * p] = bf16_lo(kp);
            kv[4 * tt + 2 * p + 1] = bf16_hi(kp);
        }
    }
    ks.beta = tok_ok ? raw.beta : 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) ks.v[c][i] = bf16_bits(raw.v[c][i]);
    }
    if (more) load_raw(raw, a, t0 + kC, b, h, off, grp, n16);

    float qb[8], kb[8], kh[8], kd[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float gam = row_prefix_sum(gv[j]);  // gamma of this lane's token, channel of slot j
        const float ep = __expf(gam);
        const float em = __builtin_amdgcn_rcpf(ep);
        ks.eC[j] = row_bcast<15>(ep);             // e^gamma_C of that channel
        qb[j] = qv[j] * ep;
        kb[j] = kv[j] * ep;
        kh[j] = kv[j] * em;
        kd[j] = kv[j] * (ks.eC[j] * em);
    }
    ks.Qb = split8(qb);
    ks.Kb = split8(kb);
    const Sp8 Kh = split8(kh), Kd = split8(kd);
    if (w == 0 && grp == 0) sm.beta[par][n16] = ks.beta;

    // Kd to "channel per lane" for the contraction over tokens
    ks.KdT[0].hi = transpose_tile(first4(Kd.hi), ident);
    ks.KdT[0].lo = transpose_tile(first4(Kd.lo), ident);
    ks.KdT[1].hi = transpose_tile(last4(Kd.hi), ident);
    ks.KdT[1].lo = transpose_tile(last4(Kd.lo), ident);

    // partial Grams over this wave's 32 channels, transposed:
    // mm32(Kh, Kb)[m][n] = Kh_m . Kb_n = (Kb Kh^T)[n][m], so lane (n, g) gets row n, columns 4g + i
    sm.gram[par][w][0][n16][grp] = mm32(Kh, ks.Kb, zero);
    sm.gram[par][w][1][n16][grp] = mm32(Kh, ks.Qb, zero);
}

// M = (I + A)^-1 diag(beta) of the chunk with parity `par` (its partial
// Grams must be visible): wave w solves columns 4w .. 4w + 3, one per 16-lane
// row.  Returns the P fragment (row n, columns 4g .. 4g + 3).
__device__ __forceinline__ f32x4 solve(Smem &sm, int par, float beta_r, int w, int grp, int n16) {
    // lane (row r = n, column group g): sum the partial Grams of row r, columns 4g .. 4g + 3
    f32x4 as = sm.gram[par][0][0][n16][grp], ps = sm.gram[par][0][1][n16][grp];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
        as += sm.gram[par][ww][0][n16][grp];
        ps += sm.gram[par][ww][1][n16][grp];
    }
    f32x4 av;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        av[i] = (4 * grp + i < n16) ? beta_r * as[i] : 0.f;
        ps[i] = (4 * grp + i <= n16) ? ps[i] : 0.f;
    }
    sm.A[w][n16][grp] = av;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float ar[kC];  // row n of A
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
        const f32x4 row = sm.A[w][n16][u4];
#pragma unroll
        for (int j = 0; j < 4; ++j) ar[4 * u4 + j] = row[j];
    }
    const int s = 4 * w + grp;  // the column this lane solves
    float x = (n16 == s) ? 1.f : 0.f;
    tri_pivots<0>(x, ar);
    sm.M[par][n16][s] = x * sm.beta[par][s];
    return ps;
}

// Partial X = Kb S0 and Y = Qb S0 over this wave's channels.
__device__ __forceinline__ void state_xy(Smem &sm, int par, const KSide &ks, const f32x4 (&Sacc)[2][2], int w,
                                         int grp, int n16) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const float sv[8] = {Sacc[0][c][0], Sacc[0][c][1], Sacc[0][c][2], Sacc[0][c][3],
                             Sacc[1][c][0], Sacc[1][c][1], Sacc[1][c][2], Sacc[1][c][3]};
        const Sp8 Sb = split8(sv);
        sm.xy[par][w][0][c][n16][grp] = mm32(ks.Kb, Sb, zero);
        sm.xy[par][w][1][c][n16][grp] = mm32(ks.Qb, Sb, zero);
    }
}

// U = M (V - X), O = scale (Y + P U) and S = diag(e^gamma_C) S0 + Kd^T U for
// the chunk starting at t0 (parity `par`).
__device__ __forceinline__ void state_update(const PrefillArgs &a, Smem &sm, int par, const KSide &ks,
                                             const f32x4 &Pfrag, int64_t t0, int64_t b, int64_t h, int col0,
                                             int w, int grp, int n16, f32x4 (&Sacc)[2][2]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const int64_t T = a.T, H = a.H;
    Sp4 Z[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        f32x4 xs = sm.xy[par][0][0][c][n16][grp];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) xs += sm.xy[par][ww][0][c][n16][grp];
        Z[c] = split4(ks.v[c] - xs);
    }
    const Sp4 Mf = split4(*reinterpret_cast<const f32x4 *>(&sm.M[par][n16][4 * grp]));
    Sp4 Uc[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) Uc[c] = split4(mm16(Mf, Z[c], zero));

    // O: waves 0 and 1 write column tiles 0 and 1
    if (w < 2) {
        f32x4 Y = sm.xy[par][0][1][w][n16][grp];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) Y += sm.xy[par][ww][1][w][n16][grp];
        const Sp4 Pf = split4(Pfrag);
        Sp4 Uw;  // select without a run-time register-array index (which would go to scratch)
        Uw.hi = (w == 0) ? Uc[0].hi : Uc[1].hi;
        Uw.lo = (w == 0) ? Uc[0].lo : Uc[1].lo;
        const f32x4 O = mm16(Pf, Uw, Y);
        char *ob = reinterpret_cast<char *>(a.o + ((b * T + t0) * H + h) * kD);  // wave uniform
        const int HD = static_cast<int>(H) * kD;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (t0 + 4 * grp + i < T)
                *reinterpret_cast<float *>(ob + 4u * static_cast<uint32_t>((4 * grp + i) * HD + col0 + 16 * w + n16)) =
                    a.scale * O[i];
        }
    }

    // S: the state rows of lane (n, g) are the channels of its operand slots,
    // so eC[j] is the decay of row 4g + j of tile 0 (j < 4) or of tile 1.
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            f32x4 s0;
#pragma unroll
            for (int i = 0; i < 4; ++i) s0[i] = ks.eC[4 * tt + i] * Sacc[tt][c][i];
            Sacc[tt][c] = mm16(ks.KdT[tt], Uc[c], s0);
        }
    }
}

__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
    __shared__ Smem sm;

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
    const int64_t T = a.T;
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
    const LaneOffsets off = lane_offsets(a.H, w, grp, n16, col0);
    if (nchunks > 0) {
        // Pipeline: iteration n runs the k-side of chunk n + 1 beside the state
        // contractions of chunk n, then the solve of chunk n + 1 beside the
        // state update of chunk n; one barrier per chunk.  The loop is unrolled
        // twice so the per-chunk registers alternate between ks[0] and ks[1]
        // without copies.
        RawChunk raw;
        load_raw(raw, a, 0, b, h, off, grp, n16);
        KSide ks[2];
        f32x4 Pf[2];
        kside(a, sm, raw, 0, nchunks > 1, b, h, off, 0, w, grp, n16, ident, ks[0]);
        __syncthreads();
        Pf[0] = solve(sm, 0, ks[0].beta, w, grp, n16);
        auto step = [&](auto cur_tag, int64_t n) {
            constexpr int CUR = decltype(cur_tag)::value, NXT = CUR ^ 1;
            const int64_t t0 = n * kC;
            const bool has_next = n + 1 < nchunks;
            state_xy(sm, CUR, ks[CUR], Sacc, w, grp, n16);
            if (has_next) kside(a, sm, raw, t0 + kC, n + 2 < nchunks, b, h, off, NXT, w, grp, n16, ident, ks[NXT]);
            __syncthreads();  // X, Y of chunk n, Grams of chunk n + 1 and M of chunk n are in LDS
            if (has_next) Pf[NXT] = solve(sm, NXT, ks[NXT].beta, w, grp, n16);
            state_update(a, sm, CUR, ks[CUR], Pf[CUR], t0, b, h, col0, w, grp, n16, Sacc);
            // No second barrier: xy[CUR] and gram[NXT] are rewritten only after
            // the next barrier, and M[NXT], written above, is read only after it.
        };
        for (int64_t n = 0; n < nchunks; n += 2) {
            step(std::integral_constant<int, 0>{}, n);
            if (n + 1 >= nchunks) break;
            step(std::integral_constant<int, 1>{}, n + 1);
        }
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
    hipLaunchKernelGGL(prefill_mfma_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
