// kda_prefill_mfma.h -- chunked KDA prefill on the gfx950 matrix cores: the
// kernel template.  kda_prefill_mfma.hip instantiates and launches the fp32
// log-decay, checkpoint and no-output variants, kda_prefill_mfma_gate.hip the
// gate-logit variants; the two are compiled with different scheduling
// strategies (each the faster one for its variants).
//
// Handles bf16 q/k/v with d_k = d_v = 128 (fp32 gates, state and output).
// One work-group per (batch, head, 32-column value slice): 4 slices per head,
// so a 56-head sequence runs on 224 work-groups, one per compute unit.  The
// slices of one head are placed on the same XCD (blockIdx -> XCD is
// round-robin), so their repeated reads of q, k, g hit that XCD's L2.
//
// Chunk form for a 16-token chunk with start state S0 (rows = key channels),
// per-channel cumulative log-decay gamma_r = g_1 + ... + g_r and
// gamma_C = gamma_16:
//   Qb = q * e^gamma      Kb = k * e^gamma      Kh = k * e^-gamma
//   A  = strict_lower(diag(beta) Kb Kh^T)        (I + A) is unit lower triangular
//   P  = lower(Qb Kh^T)
//   M  = (I + A)^-1 diag(beta)
//   X  = Kb S0,   Y = Qb S0                      (the two state contractions)
//   U  = M (V - X)
//   O  = scale * (Y + P U)
//   S  = diag(e^gamma_C) (S0 + Kh^T U)
// The last line is diag(e^gamma_C) S0 + Kd^T U with Kd = k * e^(gamma_C - gamma)
// written with the per-channel factor e^gamma_C taken out of Kd, so the
// update needs no operand of its own: the channel sum S0 + Kh^T U is formed
// in fp32 and then scaled, which keeps both terms' relative accuracy.
// The 16-token chunk with gates >= -5 keeps every e^(+-gamma) inside the bf16
// normal range, so all products can use bf16 matrix instructions (Kimi K3
// paper digest, devpress.csdn.net, section 2.1 (1)).  Each product is taken
// in three bf16 passes (x = x_hi + x_lo; a*b ~ a_hi b_hi + a_hi b_lo +
// a_lo b_hi) with fp32 accumulation, which keeps fp32-level accuracy.
//
// Work split inside a work-group: 12 waves, three per SIMD, in three roles.
//  * k-side waves 0..3 work ahead of the state: wave kw takes key channels
//    [32 kw, 32 kw + 32) of chunk n + 2 (gate prefix sums, exponentials, the
//    scaled and split operands, its partial Grams).  Everything they produce
//    goes to LDS: a ring of three chunks of operands, double-buffered Grams.
//    A translation unit may set two k-side waves per SIMD instead (16 waves;
//    waves 12..15 are the second ones): each then takes one 16-channel tile,
//    half of a quarter, and the solvers sum eight partial Grams.
//  * solver waves 8..11 sum the partial Grams of chunk n + 1 and solve
//    (I + A) M = diag(beta), four columns each, and form P (double-buffered).
//  * state waves 4..7 carry the state slice: wave (row half rh, column tile
//    ct) holds state rows [64 rh, 64 rh + 64) x columns 16 ct .. 16 ct + 15
//    in registers and runs the state part of chunk n.  The two row halves of
//    a column tile exchange their partial X, Y through LDS with a flag
//    handshake; both then form the same U for their own rows.  They read a
//    chunk's operands into registers during the step before its own, so
//    the state step waits on LDS only for M, P and the partner's partials.
// One work-group barrier per chunk hands the k-side of later chunks to the
// state waves; one wave of each role shares each SIMD.  The state waves run
// at a raised wave priority: their chain from chunk to chunk sets the pace,
// and the other two roles (which work ahead) fill the SIMD's spare issue
// cycles.
//
// Operand layouts (lane l, row group g = l / 16, n = l % 16):
//   16x16x16 (bf16_1k):  A[m = n][k = 4g + i],  B[k = 4g + i][col = n]
//   16x16x32 (bf16):     A[m = n][k = 8g + j],  B[k = 8g + j][col = n]
//   result:              C[row = 4g + i][col = n]
// q/k normalisation (the NORM variants): with c_t = 1 / max(||k_t||, eps) and
// d_t = 1 / max(||q_t||, eps) per token, the normalised operands are
// diag(c) Kb, diag(c) Kh and diag(d) Qb, and the chunk form becomes
//   A = diag(c) A0 diag(c), A0 = strict_lower(diag(beta) Kb Kh^T)
//   U' = M' (V - diag(c) Kb S0),  M' = diag(c) (I + A)^-1 diag(beta)   (U' = diag(c) U)
//   O = scale diag(d) (Y + P U')                 S = diag(e^gamma_C) (S0 + Kh^T U')
// with Kb, Kh, Qb, P, Y those of the raw q and k: no operand is rescaled.
// Since (I + D A0 D)^-1 = D^-1 (I + D^2 A0)^-1 D for D = diag(c),
//   M' = (I + diag(c^2) A0)^-1 diag(c beta):
// the solver scales row r of A0 by c_r^2 and starts column s at c_s beta_s,
// so each lane needs only the c of its own row.  ||k_t||^2 is the diagonal
// of Kb Kh^T (the decay factors cancel), which the solver sums anyway;
// ||q_t||^2 is the diagonal of one more (exact, one-pass) bf16 product of the
// raw q per k-side wave.  The state waves take c into the subtraction
// V - c X (a fused multiply-add) and scale d into o's store.
//
// "Token per lane": lane (n, g) holds token n of the chunk and, in slot j of
// an 8-wide operand of quarter kw, key channel 32 kw + 4g + j (j < 4) or
// 32 kw + 16 + 4g + j - 4 (j >= 4).  This is the operand layout of every
// contraction over channels (X, Y, the Grams); the state rows are kept in the
// result layout of 16-row tiles, which lists the same channels in the same
// slots.  q, k, g are loaded straight into it with 8- and 16-byte loads, and
// the cumulative decay over tokens is a prefix sum across the 16 lanes of a
// row (DPP row shifts).  Kh in the update, a contraction over tokens, needs
// "channel per lane" (channel n, tokens 4g .. 4g + 3): the k-side stores its
// tiles token-major and the state waves read them with gfx950's transposing
// LDS read, which delivers that layout.  The Grams are formed transposed (Kh Kb^T, Kh Qb^T), so their result layout is
// "row n, columns 4g + i", the A-operand layout of U = M Z and P U.
#pragma once

#include <cstdlib>
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
using u16x2 = unsigned short __attribute__((ext_vector_type(2)));

constexpr int kD = 128;     // head dimension (d_k = d_v)
constexpr int kDVS = 32;    // value columns per work-group
constexpr int kNV = kD / kDVS;
constexpr int kC = kChunk;  // 16
// k-side waves per SIMD, set per translation unit before this header is
// included: 1 (one 32-channel quarter per k-side wave, 12 waves) or 2 (one
// 16-channel tile per k-side wave, 16 waves: the second k-side wave of SIMD
// s is wave 12 + s).
#ifndef KDA_KSIDE_WAVES_PER_SIMD
#define KDA_KSIDE_WAVES_PER_SIMD 1
#endif
constexpr int kKSW = KDA_KSIDE_WAVES_PER_SIMD;
static_assert(kKSW == 1 || kKSW == 2, "one or two k-side waves per SIMD");
constexpr int kThreads = 768 + 256 * (kKSW - 1);
constexpr int kRing = 3;    // chunks of k-side operands in flight
constexpr float kLog2e = 1.4426950408889634f;

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

// A packed bf16 pair held in a scalar register.  The constant goes through
// an empty asm so that it is not folded into an inline constant: the
// compiler encodes the pair (-1, 0) as the inline constant -1.0 for the bf16
// dot product, and the hardware was observed to compute wrong remainders
// from that encoding (a literal or a register operand gives exact ones).
__device__ __forceinline__ bf16x2 sgpr_pair(uint32_t bits) {
    asm("" : "+s"(bits));
    return __builtin_bit_cast(bf16x2, bits);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi), both rounded to
// nearest: |x - hi - lo| <= 2^-16 |x|.  x - hi is exact in fp32; a bf16 dot
// product with (-1, 0) forms it in one instruction (-hi + x).  Per pair of
// values: one conversion packs the two hi halves, two dot products give the
// remainders, one conversion packs the two lo values.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    const bf16x2 h = __builtin_convertvector((f32x2){x0, x1}, bf16x2);
    const bf16x2 m0 = sgpr_pair(0x0000bf80u);  // (-1, 0)
    const bf16x2 m1 = sgpr_pair(0xbf800000u);  // (0, -1)
    const float l0 = __builtin_amdgcn_fdot2_f32_bf16(h, m0, x0, false);
    const float l1 = __builtin_amdgcn_fdot2_f32_bf16(h, m1, x1, false);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){l0, l1}, bf16x2));
}
// The state between steps: S holds the fp32 remainders S - hi, Shi the
// packed bf16 high halves (tile 2 js in the first four slots of Shi[js], tile
// 2 js + 1 in the last four).  state_split forms that pair from a full S,
// state_full the full value back.
__device__ __forceinline__ void state_split(f32x4 (&S)[4], bf16x8 (&Shi)[2]) {
#pragma unroll
    for (int js = 0; js < 2; ++js) {
        float sv[8] = {S[2 * js][0],     S[2 * js][1],     S[2 * js][2],     S[2 * js][3],
                       S[2 * js + 1][0], S[2 * js + 1][1], S[2 * js + 1][2], S[2 * js + 1][3]};
        uint32_t h[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const bf16x2 hh = __builtin_convertvector((f32x2){sv[2 * p], sv[2 * p + 1]}, bf16x2);
            sv[2 * p] = __builtin_amdgcn_fdot2_f32_bf16(hh, sgpr_pair(0x0000bf80u), sv[2 * p], false);
            sv[2 * p + 1] = __builtin_amdgcn_fdot2_f32_bf16(hh, sgpr_pair(0xbf800000u), sv[2 * p + 1], false);
            h[p] = __builtin_bit_cast(uint32_t, hh);
        }
        Shi[js] = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[2 * js][i] = sv[i];
            S[2 * js + 1][i] = sv[4 + i];
        }
    }
}
__device__ __forceinline__ float state_full(const f32x4 (&S)[4], const bf16x8 (&Shi)[2], int t, int i) {
    return S[t][i] + static_cast<float>(Shi[t >> 1][4 * (t & 1) + i]);
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



__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf16_bits(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// DPP data movement inside each 16-lane row.  A lane whose source lies
// outside its row (row shifts) reads 0 (bound_ctrl), which is what the prefix
// sums need and lets the move fold into the instruction that uses it.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// Right-looking forward substitution for one column of (I + A)^-1: lane
// (row r = n, group g) holds X[r][s] for one column s per 16-lane row.  At
// pivot u every row subtracts A[r][u] times row u; row u of the same column
// lives in lane u of the same 16-lane row, so a DPP broadcast replaces any LDS
// traffic.  A is strictly lower triangular, so rows r <= u are unaffected
// (A[r][u] = 0).
// `nar` holds row n of -A, so each pivot is one multiply-add with the
// broadcast as its DPP source operand.  The compiler does not fold a
// row_newbcast move into the multiply-add (it emits a separate move), so the
// fused instruction is written out; the s_nop in front gives the two wait
// states that a DPP read of a register written by the previous vector
// instruction needs, which the compiler cannot see inside the asm.
template <int U>
__device__ __forceinline__ void tri_pivots(float &x, const float (&nar)[kC]) {
    if constexpr (U < kC - 1) {
        asm("s_nop 1\n\tv_fmac_f32_dpp %0, %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
            : "+v"(x)
            : "v"(nar[U]), "i"(U));
        tri_pivots<U + 1>(x, nar);
    }
}

// Everything the state waves need of one chunk, in the lane order they read
// it (every access is lane-contiguous): one slot of the LDS ring.
struct Ops {
    bf16x8 qk[2][4][2][64];  // [Qb, Kb][32-channel quarter][hi, lo][lane], token per lane
    bf16x4 kht[8][2][64];    // [16-channel tile][hi, lo][4 token + channel / 4], Kh token-major
    f32x4 eq[2][4][4];       // e^gamma_C: [rh][g][q] holds channels 64 rh + 16 t + 4 g + q, t = 0..3
    bf16x4 Mhl[2][64];       // M = (I + A)^-1 diag(beta), split [hi, lo][lane], A-operand layout
    bf16x4 P[2][64];         // P split [hi, lo][lane]: lane (n, g) holds row n, columns 4g .. 4g + 3
    uint16_t vt[kDVS][kC];   // v of the work-group's columns, transposed: [column][token]
};

struct Smem {
    Ops ops[kRing];               // chunks n, n + 1, n + 2
    f32x4 gram[2][4 * kKSW][2][64];  // partial Grams [parity][k-side wave][A, P][lane]
    float beta[2][kC];
    f32x4 arow[4][kC][5];         // summed, masked A per solver wave; rows padded to 80 bytes
    f32x4 xy[2][2][2][64];        // partial X, Y [row half][X, Y][column tile][lane]
    uint32_t flag[2][2];          // state-wave handshake [column tile][row half]
};
// The q/k normalisation's LDS (after everything else, so the variants without
// it keep their layout).
struct NormLds {
    float qq[kRing][4 * kKSW][kC];  // partial ||q_t||^2 [ring slot][k-side wave][token]
    float f[kRing][2][kC];          // [ring slot][c, scale d][token], for the state waves
};
struct SmemNorm : Smem {
    NormLds nrm;
};

// Pacing of the four value slices of one (b, h).  They run on four compute
// units of one XCD and read the same q, k and g, so the XCD's L2 serves the
// three later readers of each line only while the slices stay within some
// twenty steps of each other; left alone they drift apart by tens of steps
// over a long sequence and then read those lines from HBM again.  Every
// kPaceEvery steps one solver wave reports its step and reads the others'
// reports (consumed one step later, so no load latency is waited for).  A
// report is up to kPaceEvery steps old when read, so a slice polls only when
// it leads a started slice of its head by more than kPaceEvery + kPaceLead
// steps by the reports, i.e. by more than kPaceLead steps at least, until it
// no longer does (at most kPaceSpin polls); the small offsets of slices that
// keep pace never cause a wait.  Reports carry the launch's epoch,
// so those of other launches never count, and the slowest slice never waits.
// The pacing only delays work: no result depends on it.
constexpr int kPaceSlots = 1 << 16;  // 4 per (b, h): launches with B H <= 16384 are paced
constexpr int kPaceEvery = 8;
constexpr int kPaceLead = 6;
constexpr int kPaceSpin = 4096;
// Per-role extras go to different SIMDs (wave w runs on SIMD w % 4): the O
// products to the state waves on SIMDs 0 and 3, P to the solver wave on SIMD
// 2, the pacing to the one on SIMD 1.
constexpr int kPSolver = 2;
constexpr int kPaceSolver = 1;
constexpr int kNormSolver = 1;  // forms the state waves' q/k normalisation factors
__device__ uint64_t g_pace[kPaceSlots];

// Reports of the slices of one (b, h): lane s < 4 reads slice s's entry.
__device__ __forceinline__ uint64_t pace_read(const uint64_t *e, int lane) {
    return lane < 4 ? __hip_atomic_load(e + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : ~0ull;
}
// Steps this slice (at step n, slice nv) leads the slowest other started slice.
__device__ __forceinline__ int64_t pace_lead(uint64_t rep, uint32_t epoch, int64_t n, int nv, int lane) {
    const bool mine = lane < 4 && lane != nv && static_cast<uint32_t>(rep >> 32) == epoch;
    const int64_t step = mine ? static_cast<int64_t>(static_cast<uint32_t>(rep)) : INT64_MAX;
    int64_t lo = INT64_MAX;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t x_lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(step), s));
        const uint32_t x_hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(step >> 32), s));
        const int64_t x = static_cast<int64_t>((static_cast<uint64_t>(x_hi) << 32) | x_lo);
        lo = x < lo ? x : lo;
    }
    return lo == INT64_MAX ? 0 : n - lo;
}

// The values (loaded by the solver waves) and o (stored by the state waves)
// go through buffer descriptors: the chunk's base address and the number of
// bytes up to its last token are wave-uniform (scalar registers), and each
// lane adds its fixed 32-bit byte offset.  In a last, partial chunk the
// offsets of tokens past the end lie beyond the descriptor's range, so the
// hardware returns zeros for those loads and drops those stores: no per-lane
// clamp or test.  Offsets stay below 2^31 bytes for the head counts this
// kernel accepts.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format

__device__ __forceinline__ Rsrc make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                            kRsrcWord3);
}

// Chunk c of one (b, h) sequence: its tokens are c kC .. c kC + rem - 1, with
// rem = kC except in the last chunk.  A [B, T, H, W] tensor's chunk starts
// c kC H W elements after the sequence's base, and its bytes up to the end of
// the last token's W elements are span_rows(c) W esz, where span_rows counts
// the rows of W elements from the chunk start: (rem - 1) H + 1.  All values
// are wave uniform and 32-bit.
struct Geom {
    int H;      // heads
    int nlast;  // index of the last chunk
    int tail;   // tokens of the last chunk, 1 .. kC
};
__device__ __forceinline__ uint32_t span_rows(const Geom &g, int c) {
    const int rem = c < g.nlast ? kC : g.tail;
    return static_cast<uint32_t>((rem - 1) * g.H + 1);
}
// The descriptor of chunk c of a tensor with W elements of esz bytes per
// (token, head), from the sequence's base address.
template <int W, int ESZ>
__device__ __forceinline__ Rsrc chunk_rsrc(const void *seq_base, const Geom &g, int c) {
    const char *p = static_cast<const char *>(seq_base) +
                    static_cast<uint64_t>(static_cast<uint32_t>(c)) *
                        (static_cast<uint32_t>(g.H) * static_cast<uint32_t>(kC * W * ESZ));
    return make_rsrc(p, span_rows(g, c) * (W * ESZ));
}

// The sequence bases of one (b, h): token 0 of each input and of o.
struct SeqBase {
    const void *q, *k, *v, *g;
    const float *beta;
    float *o;
};

// Raw inputs of one chunk for a k-side lane: q, k (4 bf16 per 16-channel
// tile) and g (4 fp32 per tile) of token n in the "token per lane" layout,
// and beta of token n.
struct KRaw {
    u32x2 q[2], k[2];
    f32x4 g[2];   // fp32 log-decay or fp32 logits
    u32x2 gx[2];  // bf16 logits
    float beta;
};

// The k-side loads q, k, g and beta with plain global loads (a wave-uniform
// chunk base plus per-lane 32-bit offsets): on this part, buffer loads of the
// same addresses hit the L2 less often when the four value slices of a head
// read them, and cost about a third more HBM reads.  In a last, partial chunk
// the token index of the offsets is clamped to the last token, so the loads
// never leave the sequence.
struct KOff {
    uint32_t tok;   // token n, channel 32 kw + 4 g (elements)
    uint32_t beta;  // token n (elements of beta)
};
__device__ __forceinline__ KOff kraw_offsets(int H, int tok, int kw, int grp) {
    return KOff{static_cast<uint32_t>(tok * H * kD + (32 / kKSW) * kw + 4 * grp), static_cast<uint32_t>(tok * H)};
}
// QS: the launch needs q (the passes without o do not read it).
template <int G, bool QS>  // GateMode
__device__ __forceinline__ void load_kraw(KRaw &r, const SeqBase &sb, const Geom &gm, int c, const KOff &full,
                                          int n16, int kw, int grp) {
    const int64_t c0 = static_cast<int64_t>(c) * (kC * gm.H);  // first token row of chunk c (wave uniform)
    KOff off = full;
    if (c == gm.nlast && gm.tail < kC) off = kraw_offsets(gm.H, min(n16, gm.tail - 1), kw, grp);
    constexpr int gsz = G == kGateLogitBf16 ? 2 : 4;
    const char *qb = static_cast<const char *>(sb.q) + 2 * kD * c0;
    const char *kb = static_cast<const char *>(sb.k) + 2 * kD * c0;
    const char *gb = static_cast<const char *>(sb.g) + gsz * kD * c0;
#pragma unroll
    for (int tt = 0; tt < 2 / kKSW; ++tt) {
        const uint32_t e = off.tok + 16u * tt;
        if constexpr (QS) r.q[tt] = *reinterpret_cast<const u32x2 *>(qb + 2u * e);
        r.k[tt] = *reinterpret_cast<const u32x2 *>(kb + 2u * e);
        if constexpr (G == kGateLogitBf16)
            r.gx[tt] = *reinterpret_cast<const u32x2 *>(gb + 2u * e);
        else
            r.g[tt] = *reinterpret_cast<const f32x4 *>(gb + 4u * e);
    }
    r.beta = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(sb.beta + c0) + 4u * off.beta);
}

// What a launch reads and writes: the full prefill, or one of the passes of
// the segmented prefill that keep only the final state (kNoOut: no o; kNoValue:
// no o and zero values, the pass that forms the transition from the identity).
// Separate instantiations, so that the full prefill carries no test for them.
enum PassMode { kFull = 0, kNoOut = 1, kNoValue = 2 };

// Values of one chunk for a state lane: token 4g + i, value column `col`,
// at byte offset vb0 + i sv (vb0 per lane, the row step sv wave uniform;
// tokens past the end read as zero).
// The values of a chunk are staged by the solver waves: solver lane (wave sv,
// lane l) holds token 4 sv + l / 16, columns 2 (l % 16) and 2 (l % 16) + 1 of
// the work-group's 32, as one dword at byte offset vb0 (tokens past the end
// read as zero), and writes them into the chunk's ring slot transposed, where
// a state lane finds its four tokens 4g .. 4g + 3 of one column in 8 bytes.
__device__ __forceinline__ uint32_t load_v2(const SeqBase &sb, const Geom &gm, int c, uint32_t vb0) {
    return __builtin_amdgcn_raw_buffer_load_b32(chunk_rsrc<kD, 2>(sb.v, gm, c), vb0, 0, 0);
}
__device__ __forceinline__ void stage_v2(Ops &op, uint32_t v2, int sv, int lane) {
    const int t = 4 * sv + (lane >> 4), c = 2 * (lane & 15);
    op.vt[c][t] = static_cast<uint16_t>(v2);
    op.vt[c + 1][t] = static_cast<uint16_t>(v2 >> 16);
}

// Unpacked inputs of one chunk for a k-side lane (channel slot j of token n).
struct KIn {
    float g[8], q[8], k[8];
    float beta;
};

// K-side, first part, for the chunk starting at t0: unpacks the raw inputs in
// `raw` (the caller reloads `raw` once the unpacked values are dead, so that
// no loaded register is copied and no wait covers a younger load).
// Tokens past the end of the sequence become identity steps: their gate is
// set to 0 and their beta to 0.  That zeroes their rows and columns of A and
// M, hence their rows of U, so their (finite) q, k and v never contribute.
// With gate logits, the log-decay g = g_min sigmoid(x) is formed here.
template <int G, bool QS>  // GateMode
__device__ __forceinline__ void kside_in(const PrefillArgs &a, const KRaw &raw, KIn &in, int c, const Geom &gm,
                                         int n16) {
    in.beta = raw.beta;
#pragma unroll
    for (int tt = 0; tt < 2 / kKSW; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (G == kGateLogDecay) {
                in.g[4 * tt + i] = raw.g[tt][i];
            } else if constexpr (G == kGateLogitF32) {
                in.g[4 * tt + i] = gate_of_logit(raw.g[tt][i], a.g_min);
            } else {
                const uint32_t p = raw.gx[tt][i >> 1];
                in.g[4 * tt + i] = gate_of_logit((i & 1) ? bf16_hi(p) : bf16_lo(p), a.g_min);
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            // (without QS, q is never loaded; its unpacked values are dead)
            const uint32_t qp = QS ? raw.q[tt][p] : 0u, kp = raw.k[tt][p];
            in.q[4 * tt + 2 * p] = bf16_lo(qp);
            in.q[4 * tt + 2 * p + 1] = bf16_hi(qp);
            in.k[4 * tt + 2 * p] = bf16_lo(kp);
            in.k[4 * tt + 2 * p + 1] = bf16_hi(kp);
        }
    }
    if (c >= gm.nlast) {  // the last chunk, or one past the end (wave-uniform test)
        if ((c - gm.nlast) * kC + n16 >= gm.tail) {
#pragma unroll
            for (int j = 0; j < 8; ++j) in.g[j] = 0.f;
            in.beta = 0.f;
        }
    }
}

// Component (n % 4) of x: in lane (n, g = n / 4) of a 16x16 product's result,
// the diagonal element (n, n).  Three selects on lane-constant masks.
__device__ __forceinline__ float diag_of(f32x4 x, int n16) {
    const float lo = (n16 & 1) ? x[1] : x[0];
    const float hi = (n16 & 1) ? x[3] : x[2];
    return (n16 & 2) ? hi : lo;
}
// x summed over the four lanes n + 16 g of each n, with gfx950's cross-row
// swaps: after v_permlane16_swap the two registers hold the values of lanes
// l and l ^ 16, after v_permlane32_swap those of lanes l and l ^ 32.  (Written
// out because the compiler folds the two results of the builtins' pair into
// one when they are added; the s_nop gives the two wait states a swap needs
// after a vector write of its operands, which the compiler cannot see here.)
__device__ __forceinline__ float row_group_sum(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    float c = a + b, d = c;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(d));
    return c + d;
}
// ||q_t||^2 over this k-side wave's channels: the diagonal of the raw q's Gram
// (bf16 products are exact in fp32), one product on the loaded registers.
__device__ __forceinline__ void kside_qq(float (&qq)[4 * kKSW][kC], const KRaw &raw, int kw, int grp, int n16) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 gq;
    if constexpr (kKSW == 1) {
        const bf16x8 qr = __builtin_bit_cast(bf16x8, u32x4{raw.q[0][0], raw.q[0][1], raw.q[1][0], raw.q[1][1]});
        gq = mfma32(qr, qr, zero);
    } else {
        const bf16x4 qr = __builtin_bit_cast(bf16x4, raw.q[0]);
        gq = mfma16(qr, qr, zero);
    }
    if (grp == (n16 >> 2)) qq[kw][n16] = diag_of(gq, n16);
}

// K-side, second part: this quarter's operands of the chunk go to `op` (LDS or
// a shared slot in global memory), its partial Grams to `gr`, beta to `bt`.
// Without QS (no o) neither Qb nor P is formed.
template <bool QS>
__device__ __forceinline__ void kside(Ops &op, f32x4 (&gr)[4 * kKSW][2][64], float (&bt)[kC], const KIn &in, int kw,
                                      int grp, int n16, int lane) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const float(&gv)[8] = in.g;
    const float(&qv)[8] = in.q;
    const float(&kv)[8] = in.k;
    // log2 of the cumulative decay: 8 independent prefix sums over the
    // tokens, written shift-major so that each DPP read finds its source
    // written several instructions earlier (no hazard stalls)
    float gam[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        gam[j] = gv[j] * kLog2e;
        asm("" : "+v"(gam[j]));  // keeps gam + dpp(gam) a DPP add (not a product folded into an fma)
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) gam[j] += dpp_move<0x111>(gam[j]);  // row_shr:1
#pragma unroll
    for (int j = 0; j < 8; ++j) gam[j] += dpp_move<0x112>(gam[j]);  // row_shr:2
#pragma unroll
    for (int j = 0; j < 8; ++j) gam[j] += dpp_move<0x114>(gam[j]);  // row_shr:4
#pragma unroll
    for (int j = 0; j < 8; ++j) gam[j] += dpp_move<0x118>(gam[j]);  // row_shr:8
    float ep[8], em[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        ep[j] = __builtin_amdgcn_exp2f(gam[j]);
        em[j] = __builtin_amdgcn_exp2f(-gam[j]);
    }
    float qb[8], kb[8], kh[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        qb[j] = qv[j] * ep[j];
        kb[j] = kv[j] * ep[j];
        kh[j] = kv[j] * em[j];
    }
    // (without QS, Qb is never stored or used, so its products and split
    // are dead code)
    const Sp8 Qb = split8(qb), Kb = split8(kb), Kh = split8(kh);
    if constexpr (QS) {
        op.qk[0][kw][0][lane] = Qb.hi;
        op.qk[0][kw][1][lane] = Qb.lo;
    }
    op.qk[1][kw][0][lane] = Kb.hi;
    op.qk[1][kw][1][lane] = Kb.lo;
    // Kh tiles token-major: token n, channels 4g .. 4g + 3 of the tile at
    // 8-byte index 4n + g (the state waves transpose them as they read them)
    op.kht[2 * kw][0][4 * n16 + grp] = first4(Kh.hi);
    op.kht[2 * kw][1][4 * n16 + grp] = first4(Kh.lo);
    op.kht[2 * kw + 1][0][4 * n16 + grp] = last4(Kh.hi);
    op.kht[2 * kw + 1][1][4 * n16 + grp] = last4(Kh.lo);
    if (n16 == kC - 1) {
        // the last token's e^gamma is e^gamma_C.  Slots j < 4 of row g are
        // channels 32 kw + 4 g + j, i.e. row half kw / 2, tile t = 2 (kw % 2),
        // q = j; slots j >= 4 the same q in tile t + 1
#pragma unroll
        for (int q = 0; q < 4; ++q) reinterpret_cast<f32x2 *>(&op.eq[kw >> 1][grp][q])[kw & 1] = f32x2{ep[q], ep[q + 4]};
    }
    if (kw == 0 && grp == 0) bt[n16] = in.beta;
    // partial Grams over this quarter, transposed:
    // mm32(Kh, Kb)[m][n] = Kh_m . Kb_n = (Kb Kh^T)[n][m], so lane (n, g) gets row n, columns 4g + i
    gr[kw][0][lane] = mm32(Kh, Kb, zero);
    if constexpr (QS) gr[kw][1][lane] = mm32(Kh, Qb, zero);
}

// K-side with two k-side waves per SIMD: this wave's 16-channel tile kt (the
// half kt % 2 of the quarter kt / 2) goes to `op` as slots
// 4 (kt % 2) .. 4 (kt % 2) + 3 of the quarter's 8-wide operands (one 8-byte
// write each), its partial Grams (over 16 channels) to `gr[kt]`.  The
// unpacked inputs are the first four slots of `in`.
template <bool QS>
__device__ __forceinline__ void kside_tile(Ops &op, f32x4 (&gr)[4 * kKSW][2][64], float (&bt)[kC], const KIn &in,
                                           int kt, int grp, int n16, int lane) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    float gam[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        gam[j] = in.g[j] * kLog2e;
        asm("" : "+v"(gam[j]));  // keeps gam + dpp(gam) a DPP add (not a product folded into an fma)
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) gam[j] += dpp_move<0x111>(gam[j]);  // row_shr:1
#pragma unroll
    for (int j = 0; j < 4; ++j) gam[j] += dpp_move<0x112>(gam[j]);  // row_shr:2
#pragma unroll
    for (int j = 0; j < 4; ++j) gam[j] += dpp_move<0x114>(gam[j]);  // row_shr:4
#pragma unroll
    for (int j = 0; j < 4; ++j) gam[j] += dpp_move<0x118>(gam[j]);  // row_shr:8
    f32x4 ep, em, qb, kb, kh;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ep[j] = __builtin_amdgcn_exp2f(gam[j]);
        em[j] = __builtin_amdgcn_exp2f(-gam[j]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        qb[j] = in.q[j] * ep[j];
        kb[j] = in.k[j] * ep[j];
        kh[j] = in.k[j] * em[j];
    }
    const Sp4 Qb = split4(qb), Kb = split4(kb), Kh = split4(kh);
    const int kq = kt >> 1, half = kt & 1;
    if constexpr (QS) {
        reinterpret_cast<bf16x4 *>(&op.qk[0][kq][0][lane])[half] = Qb.hi;
        reinterpret_cast<bf16x4 *>(&op.qk[0][kq][1][lane])[half] = Qb.lo;
    }
    reinterpret_cast<bf16x4 *>(&op.qk[1][kq][0][lane])[half] = Kb.hi;
    reinterpret_cast<bf16x4 *>(&op.qk[1][kq][1][lane])[half] = Kb.lo;
    op.kht[kt][0][4 * n16 + grp] = Kh.hi;
    op.kht[kt][1][4 * n16 + grp] = Kh.lo;
    if (n16 == kC - 1) {
        // e^gamma_C: slot j of row g is channel 16 kt + 4 g + j: row half kt / 4, tile kt % 4, q = j
#pragma unroll
        for (int q = 0; q < 4; ++q) reinterpret_cast<float *>(&op.eq[kt >> 2][grp][q])[kt & 3] = ep[q];
    }
    if (kt == 0 && grp == 0) bt[n16] = in.beta;
    // partial Grams over this tile, transposed (16x16x16 products: the same
    // result layout as the quarter's 16x16x32 ones)
    gr[kt][0][lane] = mm16(Kh, Kb, zero);
    if constexpr (QS) gr[kt][1][lane] = mm16(Kh, Qb, zero);
}

// M = (I + A)^-1 diag(beta) and P of the chunk whose Grams sit in the `par`
// buffers: solver wave kw solves columns 4 kw .. 4 kw + 3, one per 16-lane row.
// NORM: c comes from the diagonal of the summed Gram, ||q||^2 from the k-side
// partials in nl->qq[slot]; row r of A is scaled by c_r^2 and column s starts
// at c_s beta_s (which gives diag(c) M), and solver kNormSolver leaves c and
// scale d in nl->f[slot].
template <bool QS, bool NORM>
__device__ __forceinline__ void solve(const f32x4 (&gr)[4 * kKSW][2][64], const float (&bt)[kC], f32x4 (&arow)[kC][5],
                                      bf16x4 (&Mo)[2][64], bf16x4 (&Po)[2][64], int kw, int grp, int n16,
                                      int lane, NormLds *nl, int slot, float eps2, float scale) {
    // lane (row r = n, column group g): sum the partial Grams of row r, columns 4g .. 4g + 3
    f32x4 as = gr[0][0][lane];
#pragma unroll
    for (int ww = 1; ww < 4 * kKSW; ++ww) as += gr[ww][0][lane];
    const float nbeta_r = -bt[n16];
    f32x4 av;  // row r of -A
    float cr = 1.f;  // NORM: c of this lane's row
    if constexpr (NORM) {
        // (Kb Kh^T)[t][t] = ||k_t||^2 sits in lane (t, t / 4), component t % 4;
        // the sum over the row groups brings it to every lane (t, g)
        const bool dlane = grp == (n16 >> 2);
        cr = norm_factor(row_group_sum(dlane ? diag_of(as, n16) : 0.f), eps2);
        const float nbc = nbeta_r * (cr * cr);
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = (4 * grp + i < n16) ? nbc * as[i] : 0.f;
        if (kw == kNormSolver && dlane) {
            float sq = nl->qq[slot][0][n16];
#pragma unroll
            for (int ww = 1; ww < 4 * kKSW; ++ww) sq += nl->qq[slot][ww][n16];
            nl->f[slot][0][n16] = cr;
            nl->f[slot][1][n16] = scale * norm_factor(sq, eps2);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = (4 * grp + i < n16) ? nbeta_r * as[i] : 0.f;
    }
    arow[n16][grp] = av;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float nar[kC];  // row n of -A
#pragma unroll
    for (int u4 = 0; u4 < 4; ++u4) {
        const f32x4 row = arow[n16][u4];
#pragma unroll
        for (int j = 0; j < 4; ++j) nar[4 * u4 + j] = row[j];
    }
    const int s = 4 * kw + grp;  // the column this lane solves
    float x = (n16 == s) ? (NORM ? bt[s] * cr : 1.f) : 0.f;  // NORM: c_s beta_s (cr = c_s in row s)
    tri_pivots<0>(x, nar);
    // M[n][s] goes to slot s % 4 = grp of lane 16 (s / 4) + n = 16 kw + n of
    // the A operand of U = M Z, as a hi/lo bf16 pair
    const float m = NORM ? x : x * bt[s];
    const __bf16 mh = static_cast<__bf16>(m);
    const __bf16 ml = static_cast<__bf16>(m - static_cast<float>(mh));
    reinterpret_cast<__bf16 *>(&Mo[0][16 * kw + n16])[grp] = mh;
    reinterpret_cast<__bf16 *>(&Mo[1][16 * kw + n16])[grp] = ml;
    // P (lower triangle with the diagonal) comes from one solver wave alone
    if (QS && kw == kPSolver) {
        f32x4 ps = gr[0][1][lane];
#pragma unroll
        for (int ww = 1; ww < 4 * kKSW; ++ww) ps += gr[ww][1][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) ps[i] = (4 * grp + i <= n16) ? ps[i] : 0.f;
        const Sp4 pp = split4(ps);  // stored split: the state waves use it as is
        Po[0][lane] = pp.hi;
        Po[1][lane] = pp.lo;
    }
}

// Operands of one chunk that a state wave holds in registers.  They are read
// during the step before their own (the k-side finished them one step before
// that): Kb and Qb once that step's X and Y are formed, Kh^T and e^gamma_C
// once its update has consumed its own.  The reads then have a whole step
// to land, and the state step itself waits only for M and P.
struct SOps {
    Sp8 Kb[2], Qb[2];  // channels of quarters 2 rh + js, operand layout
    Sp4 KhT[4];        // 16-channel tiles 4 rh + t, channel per lane
    f32x4 eq;          // e^gamma_C of channels 64 rh + 16 t + 4 g + (n & 3), t = 0..3
};
template <bool QS>
__device__ __forceinline__ void read_kq(SOps &s, const Ops &op, int rh, int lane) {
#pragma unroll
    for (int js = 0; js < 2; ++js) {
        s.Kb[js] = Sp8{op.qk[1][2 * rh + js][0][lane], op.qk[1][2 * rh + js][1][lane]};
        if constexpr (QS) s.Qb[js] = Sp8{op.qk[0][2 * rh + js][0][lane], op.qk[0][2 * rh + js][1][lane]};
    }
}
// Transposing LDS read (gfx950): inside each group of 16 lanes, lane i
// receives in slot k the element (i mod 4) of the 8 bytes addressed by lane
// i / 4 + 4 k.  Over a token-major 16 x 16 tile (token r, channel c at element
// 16 r + c), with every lane addressing its own 8-byte index, lane (n, g)
// receives channel n of tokens 4g .. 4g + 3: the A operand of Kh^T U.
__device__ __forceinline__ bf16x4 read_tr(const bf16x4 *p) {
    using lds_s16x4 = __attribute__((address_space(3))) s16x4;
    return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p)));
}
__device__ __forceinline__ void read_kh(SOps &s, const Ops &op, int rh, int grp, int n16, int lane) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
        s.KhT[t] = Sp4{read_tr(&op.kht[4 * rh + t][0][lane]), read_tr(&op.kht[4 * rh + t][1][lane])};
    s.eq = op.eq[rh][grp][n16 & 3];
}
// lane I of each group of four lanes, to the whole group (DPP quad_perm [I, I, I, I])
template <int I>
__device__ __forceinline__ float quad_bcast(float x) {
    return dpp_move<I * 0x55>(x);
}

// State part of chunk n for state wave (rh, ct): X, Y, U, O and
// the state update S = diag(e^gamma_C) (S0 + Kh^T U) of this wave's rows.
// `op` is chunk n's ring slot (M, P are read from it here; the rest is in
// `cur`), `nx` chunk n + 1's, whose operands are read into `nxt`.
// NORM: nf holds the chunk's normalisation factors (c and scale d of token t
// in nf[0][t], nf[1][t]); M arrives as diag(c) M.
template <int MODE, bool NORM>
__device__ __forceinline__ void state_chunk(const PrefillArgs &a, Smem &sm, const Ops &op, const Ops &nx, int64_t n,
                                            const SeqBase &sb, const Geom &gm, f32x4 (&S)[4], bf16x8 (&Shi)[2],
                                            const SOps &cur, SOps &nxt, int rh, int ct, int grp, int n16, int lane,
                                            uint32_t ob0, uint32_t so, bf16x4 ident, const float (*nf)[kC]) {
    constexpr bool QS = MODE == kFull;  // Y and O only where o is written
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const Sp4 Mf = Sp4{op.Mhl[0][lane], op.Mhl[1][lane]};
    const Sp4 Pf = Sp4{op.P[0][lane], op.P[1][lane]};
    f32x4 ck = zero, osc = zero;  // NORM: c and scale d of tokens 4g + i
    if constexpr (NORM) {
        ck = *reinterpret_cast<const f32x4 *>(&nf[0][4 * grp]);
        osc = *reinterpret_cast<const f32x4 *>(&nf[1][4 * grp]);
    }
    // this chunk's values are read with M and P, ahead of the handshake: LDS
    // reads complete in order, so a read issued after the handshake would
    // also wait for the next chunk's operand reads issued there
    u32x2 vp = {0u, 0u};
    if constexpr (MODE != kNoValue) vp = *reinterpret_cast<const u32x2 *>(&op.vt[16 * ct + (lane & 15)][4 * grp]);

    // partial X = Kb S0 and Y = Qb S0 over this wave's 64 channels; the state
    // rows of tiles 2js, 2js + 1 are the channels of operand slots 0..3, 4..7.
    // S0 arrives split (S0 - hi in S, hi packed in Shi, from the end of the
    // previous step); the update adds hi back with an identity product.
    f32x4 X = zero, Y = zero;
#pragma unroll
    for (int js = 0; js < 2; ++js) {
        uint32_t l[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int t = 2 * js + (p >> 1), i = 2 * (p & 1);
            l[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){S[t][i], S[t][i + 1]}, bf16x2));
        }
        const Sp8 Sb{Shi[js], __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]})};
        X = mm32(cur.Kb[js], Sb, X);
        if constexpr (QS) Y = mm32(cur.Qb[js], Sb, Y);
    }
    // the row half rh == ct forms O of column tile ct (waves 4 and 7, on
    // SIMDs 0 and 3); the other half hands it its Y
    const bool owave = rh == ct;
    sm.xy[rh][0][ct][lane] = X;
    if (QS && !owave) sm.xy[rh][1][ct][lane] = Y;
    // Y is formed here in both halves (so that Qb dies before the next
    // chunk's operands land in other registers)
    if constexpr (QS) asm volatile("" ::"v"(Y));
    // hand the partials to the other row half of this column tile and wait
    // for its own: its flag reaches n + 1 in this chunk and cannot move
    // further before the next work-group barrier
    const uint32_t tag = static_cast<uint32_t>(n + 1);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __hip_atomic_store(&sm.flag[ct][rh], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    // (a poll is one LDS round trip; the partner is at most a few hundred
    // cycles away, so the loop does not sleep between polls)
    while (__hip_atomic_load(&sm.flag[ct][rh ^ 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != tag) {
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const f32x4 Xo = sm.xy[rh ^ 1][0][ct][lane];
    f32x4 Yo = zero;  // the other half's Y (used by the O wave)
    if constexpr (QS) Yo = sm.xy[rh ^ 1][1][ct][lane];
    // the next chunk's Kb, Qb replace this chunk's (dead after X, Y); issued
    // after the handshake so that no flag poll waits for them
    asm volatile("" ::: "memory");
    read_kq<QS>(nxt, nx, rh, lane);
    X += Xo;

    f32x4 vv = zero;
    if constexpr (MODE != kNoValue) {
        vv[0] = __uint_as_float(vp[0] << 16);
        vv[1] = __uint_as_float(vp[0] & 0xffff0000u);
        vv[2] = __uint_as_float(vp[1] << 16);
        vv[3] = __uint_as_float(vp[1] & 0xffff0000u);
    }
    // NORM: V - diag(c) Kb S0, and M = diag(c) M gives U' = diag(c) U, which
    // the update and P U' then take with the raw Kh and P
    const f32x4 Z = NORM ? vv - ck * X : vv - X;
    const Sp4 U = split4(mm16(Mf, split4(Z), zero));

    if (owave && MODE == kFull) {
        const f32x4 O = mm16(Pf, U, Y + Yo);
        // o has the layout of v: token 4g + i, column `col` at byte offset ob0 + i so
        const Rsrc ro = chunk_rsrc<kD, 4>(sb.o, gm, static_cast<int>(n));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, (NORM ? osc[i] : a.scale) * O[i]), ro,
                                                  ob0, i * so, 0);
    }

    // S: lane (n, g) holds rows 4g + i of tile t, channel 64 rh + 16 t + 4 g + i,
    // whose e^gamma_C sits in component t of lane (4 (n / 4) + i, g)'s eq
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bf16x4 hi = t & 1 ? last4(Shi[t >> 1]) : first4(Shi[t >> 1]);
        const f32x4 acc = mm16(cur.KhT[t], U, mfma16(ident, hi, S[t]));  // S0 = hi + (S0 - hi)
        S[t][0] = quad_bcast<0>(cur.eq[t]) * acc[0];
        S[t][1] = quad_bcast<1>(cur.eq[t]) * acc[1];
        S[t][2] = quad_bcast<2>(cur.eq[t]) * acc[2];
        S[t][3] = quad_bcast<3>(cur.eq[t]) * acc[3];
    }
    // the next step's split of S happens here, at the end of this step
    state_split(S, Shi);
    // the update is issued before the next chunk's Kh^T, e^gamma_C are read
    asm volatile("" ::"v"(S[0]), "v"(S[1]), "v"(S[2]), "v"(S[3]) : "memory");
    read_kh(nxt, nx, rh, grp, n16, lane);
}

// The step sequence of a work-group over nchunks chunks, with one barrier
// after each step.  Step n runs body(parity, solve, kside, state, n), where
// the three flags (compile-time) say whether chunk n + 1 is solved, chunk
// n + 2 prepared and chunk n advanced: steps -2 and -1 fill the pipeline,
// the last two drain it, and every step in between does all three.  Both
// roles call this with the same nchunks, so they meet the same barriers.
// The barrier that ends a step.  A role whose LDS writes others read in the
// next step (k-side, solver) waits for its LDS operations first
// (__syncthreads).  The state waves publish nothing through the barrier
// (their X, Y exchange has its own flags), and their loads in flight are read
// ahead of the slot's reuse: they arrive at the barrier without waiting.  The
// empty asm statements keep the compiler from moving LDS accesses across it.
template <bool FENCE>
__device__ __forceinline__ void step_barrier() {
    if constexpr (FENCE) {
        __syncthreads();
    } else {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

template <bool FENCE = true, class Body>
__device__ __forceinline__ void run_steps(int64_t nchunks, Body &&body) {
    using F = std::false_type;
    using Tr = std::true_type;
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    if (nchunks <= 0) return;
    // steps -2 and -1 always run the k-side (with one chunk, step -1 prepares
    // a chunk past the end whose tokens are all masked and whose operands
    // are never read): the same load pattern on every path keeps the
    // compiler's load-count bookkeeping exact at the loop entry
    body(P0{}, F{}, Tr{}, F{}, -2);  // k-side of chunk 0
    step_barrier<FENCE>();
    body(P1{}, Tr{}, Tr{}, F{}, -1);  // solve of chunk 0, k-side of chunk 1
    step_barrier<FENCE>();
    // steps 0 .. nchunks - 3 do all three; the loop ends on an odd step, so
    // every step after it has a parity known here (no register buffer has
    // to survive a step whose parity is decided at run time)
    int64_t n = 0;
    for (; n + 1 < nchunks - 2; n += 2) {  // chunks n + 2 and n + 3 exist
        body(P0{}, Tr{}, Tr{}, Tr{}, n);
        step_barrier<FENCE>();
        body(P1{}, Tr{}, Tr{}, Tr{}, n + 1);
        step_barrier<FENCE>();
    }
    if (nchunks & 1) {  // n = nchunks - 3 (or nchunks = 1: n = 0 is the last step)
        if (nchunks > 1) {
            body(P0{}, Tr{}, Tr{}, Tr{}, n);
            step_barrier<FENCE>();
            body(P1{}, Tr{}, F{}, Tr{}, n + 1);  // solve of the last chunk
            step_barrier<FENCE>();
            n += 2;
        }
        body(P0{}, F{}, F{}, Tr{}, n);
        step_barrier<FENCE>();
    } else {  // n = nchunks - 2
        body(P0{}, Tr{}, F{}, Tr{}, n);  // solve of the last chunk
        step_barrier<FENCE>();
        body(P1{}, F{}, F{}, Tr{}, n + 1);
        step_barrier<FENCE>();
    }
}

// The kernel body.  CKPT: the launch writes state checkpoints (a separate
// instantiation, so the plain prefill carries no test for it).  MODE: a
// PassMode.  NORM: q and k are normalised (with kFull only).
template <bool CKPT, int G, int MODE, bool NORM>  // G: GateMode
__device__ __forceinline__ void prefill_mfma_body(PrefillArgs a) {
    static_assert(!NORM || MODE == kFull, "the q/k normalisation comes with the full prefill only");
    __shared__ std::conditional_t<NORM, SmemNorm, Smem> sm;
    constexpr bool QS = MODE == kFull;  // q, Qb, P and Y are needed only where o is written

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    if (bh >= BH) return;  // padding blocks of the last XCD round (whole work-group)
    const int64_t b = bh / a.H, h = bh % a.H;
    const int64_t T = a.T;
    const int64_t nchunks = (T + kC - 1) / kC;
    const int col0 = nv * kDVS;
    const int64_t sbase = bh * kD * kD;

    const bool kwave = w < 4 || (kKSW == 2 && w >= 12);
    const bool swave = w >= 4 && w < 8;
    // k-side role: channel quarter (one k-side wave per SIMD) or 16-channel tile (two)
    const int kw = kKSW == 1 ? w : (w < 4 ? 2 * w : 2 * (w - 12) + 1);
    const int rh = (w - 4) >> 1;   // state role: row half
    const int ct = (w - 4) & 1;    //             column tile
    const int sv = w - 8;          // solver role: columns 4 sv .. 4 sv + 3
    const int col = col0 + 16 * ct + n16;

    if (tid < 4) (&sm.flag[0][0])[tid] = 0u;

    const KOff koff = kraw_offsets(static_cast<int>(a.H), n16, kw, grp);
    // a state lane's token 4 grp + i, column col of o: element offset
    // voff0 + i HD within a chunk (the row step HD is wave uniform)
    const uint32_t HD = static_cast<uint32_t>(a.H) * kD;
    const uint32_t voff0 = static_cast<uint32_t>(4 * grp) * HD + static_cast<uint32_t>(col);
    // a solver lane's dword of v: token 4 sv + lane / 16, columns col0 + 2 (lane % 16) + {0, 1}
    const uint32_t vb0 = 2u * (static_cast<uint32_t>(4 * sv + (lane >> 4)) * HD +
                               static_cast<uint32_t>(col0 + 2 * (lane & 15)));
    const int64_t seq_row = b * T * a.H + h;  // token 0 of this (b, h), in rows of kD elements
    const SeqBase sb{static_cast<const uint16_t *>(a.q) + seq_row * kD, static_cast<const uint16_t *>(a.k) + seq_row * kD,
                     static_cast<const uint16_t *>(a.v) + seq_row * kD,
                     static_cast<const char *>(a.g) + (G == kGateLogitBf16 ? 2 : 4) * (seq_row * kD),
                     a.beta + seq_row, a.o ? a.o + seq_row * kD : nullptr};
    const int nlast = static_cast<int>(nchunks) - 1;
    const Geom gm{static_cast<int>(a.H), nlast, static_cast<int>(T - static_cast<int64_t>(nlast) * kC)};
    KRaw raw[2];
    f32x4 S[4];  // state rows 64 rh + 16 t + 4 g + i, column `col` (between steps: S - hi)
    bf16x8 Shi[2];  // and its high halves (between steps)

    if (kwave) {
        if (nchunks > 0) {
            load_kraw<G, QS>(raw[0], sb, gm, 0, koff, n16, kw, grp);
            load_kraw<G, QS>(raw[1], sb, gm, min(1, nlast), koff, n16, kw, grp);
        }
    } else if (swave) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 64 * rh + 16 * t + 4 * grp + i;
                S[t][i] = a.h0 ? a.h0[sbase + row * kD + col] : 0.f;
            }
        }
        state_split(S, Shi);
    }

    // Step n: the k-side waves prepare chunk n + 2, the solver waves solve
    // chunk n + 1, the state waves run chunk n; one barrier ends the step.
    // Each role runs its own copy of the step sequence, so the register
    // double-buffers of one role never meet another's in a loop phi, and
    // loaded values are consumed in the registers they land in.
    if (kwave) {
        int kslot = 0;  // ring slot of chunk n + 2
        run_steps(nchunks, [&](auto par_tag, auto, auto kside_tag, auto, int64_t n) {
            constexpr int PAR = decltype(par_tag)::value;  // n & 1
            // reload the raw buffer at the end, once the unpacked values are dead
            KIn in;
            if constexpr (decltype(kside_tag)::value) kside_in<G, QS>(a, raw[PAR], in, static_cast<int>(n) + 2, gm, n16);
            if constexpr (decltype(kside_tag)::value) {
                if constexpr (NORM) kside_qq(sm.nrm.qq[kslot], raw[PAR], kw, grp, n16);
                if constexpr (kKSW == 1)
                    kside<QS>(sm.ops[kslot], sm.gram[PAR], sm.beta[PAR], in, kw, grp, n16, lane);
                else
                    kside_tile<QS>(sm.ops[kslot], sm.gram[PAR], sm.beta[PAR], in, kw, grp, n16, lane);
                load_kraw<G, QS>(raw[PAR], sb, gm, min(static_cast<int>(n) + 4, nlast), koff, n16, kw, grp);
            }
            kslot = (kslot == kRing - 1) ? 0 : kslot + 1;
        });
    } else if (!swave) {
        int vslot = 2;  // ring slot of chunk n + 1 (n = -2 maps to slot 2)
        uint32_t v2 = 0;  // this lane's values of chunk n + 1, loaded one step ahead
        if (MODE != kNoValue && nchunks > 0) v2 = load_v2(sb, gm, 0, vb0);
        // one solver wave (kPaceSolver) paces this slice against the other slices of its (b, h)
        const bool pace = a.epoch != 0 && sv == kPaceSolver && BH * kNV <= kPaceSlots;
        uint64_t *pace_e = g_pace + (pace ? bh * kNV : 0);
        uint64_t rep = ~0ull;  // the reports read at the last report step
        run_steps(nchunks, [&](auto par_tag, auto solve_tag, auto, auto, int64_t n) {
            constexpr int PAR = decltype(par_tag)::value;  // n & 1
            if constexpr (decltype(solve_tag)::value) {
                if constexpr (MODE != kNoValue) stage_v2(sm.ops[vslot], v2, sv, lane);
                if (pace && n % kPaceEvery == 1) {
                    int64_t lead = pace_lead(rep, a.epoch, n, nv, lane);
                    for (int spin = 0; lead > kPaceEvery + kPaceLead && spin < kPaceSpin; ++spin) {
                        __builtin_amdgcn_s_sleep(4);
                        lead = pace_lead(pace_read(pace_e, lane), a.epoch, n, nv, lane);
                    }
                }
                // the reports are read before this step's value load, so the
                // next step's wait for those values covers them as well
                if (pace && n % kPaceEvery == 0) {
                    if (lane == 0)
                        __hip_atomic_store(pace_e + nv, (static_cast<uint64_t>(a.epoch) << 32) | static_cast<uint32_t>(n),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    rep = pace_read(pace_e, lane);
                }
                if constexpr (MODE != kNoValue) v2 = load_v2(sb, gm, min(static_cast<int>(n) + 2, nlast), vb0);
                NormLds *nl = nullptr;
                if constexpr (NORM) nl = &sm.nrm;
                solve<QS, NORM>(sm.gram[PAR ^ 1], sm.beta[PAR ^ 1], sm.arow[sv], sm.ops[vslot].Mhl, sm.ops[vslot].P,
                                sv, grp, n16, lane, nl, vslot, a.qk_eps2, a.scale);
            }
            vslot = (vslot == kRing - 1) ? 0 : vslot + 1;
        });
    } else {
        // the state waves carry the serial chain from chunk to chunk: the
        // SIMD issues their instructions first, and the k-side and solver
        // waves (which work ahead) fill the remaining issue cycles
        __builtin_amdgcn_s_setprio(3);
        // the 16 x 16 identity as an A operand: lane (m, kg) holds row m, columns 4 kg .. 4 kg + 3
        bf16x4 ident;
#pragma unroll
        for (int j = 0; j < 4; ++j) ident[j] = static_cast<__bf16>(n16 == 4 * grp + j ? 1.f : 0.f);
        int sslot = 1;        // ring slot of chunk n (n = -2 maps to slot 1)
        SOps so[2];           // operands of the chunks of even and odd steps
        int64_t ck_left = a.ckpt_every, ck_i = 0;  // chunks to the next checkpoint, its index
        run_steps<false>(nchunks, [&](auto par_tag, auto, auto, auto state_tag, int64_t n) {
            constexpr int PAR = decltype(par_tag)::value;
            const int nslot = (sslot == kRing - 1) ? 0 : sslot + 1;  // chunk n + 1
            if constexpr (decltype(state_tag)::value) {
                const float(*nf)[kC] = nullptr;
                if constexpr (NORM) nf = sm.nrm.f[sslot];
                state_chunk<MODE, NORM>(a, sm, sm.ops[sslot], sm.ops[nslot], n, sb, gm, S, Shi, so[PAR], so[PAR ^ 1],
                                        rh, ct, grp, n16, lane, 4u * voff0, 4u * HD, ident, nf);
                if (CKPT && --ck_left == 0) {  // the state after (ck_i + 1) * ckpt_every chunks
                    if (ck_i < a.n_ckpt) {
                        float *ck = a.ckpt + ck_i * (BH * kD * kD) + sbase;
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                ck[(64 * rh + 16 * t + 4 * grp + i) * kD + col] = state_full(S, Shi, t, i);
                        }
                    }
                    ++ck_i;
                    ck_left = a.ckpt_every;
                }
            } else if constexpr (PAR == 1) {
                // step -1: chunk 0 was prepared in step -2; read its operands for step 0
                read_kq<QS>(so[0], sm.ops[nslot], rh, lane);
                read_kh(so[0], sm.ops[nslot], rh, grp, n16, lane);
            }
            sslot = nslot;
        });
    }

    if (swave && a.hT) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 64 * rh + 16 * t + 4 * grp + i;
                a.hT[sbase + row * kD + col] = state_full(S, Shi, t, i);
            }
        }
    }
}

template <bool CKPT, int G, int MODE>  // G: GateMode
__global__ __launch_bounds__(kThreads) void prefill_mfma_kernel(PrefillArgs a) {
    prefill_mfma_body<CKPT, G, MODE, false>(a);
}
// The prefill with the q/k normalisation (a kernel of its own name, so that
// kernel traces tell it from the plain one).
template <int G>  // GateMode
__global__ __launch_bounds__(kThreads) void prefill_mfma_qknorm_kernel(PrefillArgs a) {
    prefill_mfma_body<false, G, kFull, true>(a);
}

}  // namespace

}  // namespace kda
