// kda_f32mfma.h -- building blocks of the chunk kernels that run on the fp32
// matrix cores (16x16x4 products with fp32 inputs and accumulation): tile
// products with operands read from LDS, DPP lane moves, the forward
// substitution of a unit lower-triangular 16 x 16 system, bounded buffer
// accesses and an LDS-only work-group barrier.  Used by the backward pass
// (kda_bwd.hip) and the fp32 prefill at d = 128 (kda_prefill_f32.hip).
#pragma once

#include "kda_internal.h"

namespace kda {
namespace {

// x of another lane, moved by DPP (CTRL); lanes whose source is out of range
// read 0
template <int CTRL>
__device__ __forceinline__ float dpp_mv(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

using f32x4 = float __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float x, float y, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, c, 0, 0, 0);
}

// c + A B for one 16 x 16 tile over K (a multiple of 4), A(r, k) =
// pa[r sar + k sak] and B(k, j) = pb[k sbk + j sbc].  Lane l supplies A(l % 16,
// k0 + l / 16) and B(k0 + l / 16, l % 16) to each step; component i of the
// result is C(4 (l / 16) + i, l % 16).
template <int K>
__device__ __forceinline__ f32x4 tile_mm(const float *pa, int sar, int sak, const float *pb, int sbk, int sbc, f32x4 c,
                                         int lane) {
    const int r = lane & 15, kq = lane >> 4;
    float av[K / 4], bv[K / 4];  // every operand is read before the first product
#pragma unroll
    for (int m = 0; m < K / 4; ++m) {
        av[m] = pa[r * sar + (4 * m + kq) * sak];
        bv[m] = pb[(4 * m + kq) * sbk + r * sbc];
    }
#pragma unroll
    for (int m = 0; m < K / 4; ++m) c = mfma4(av[m], bv[m], c);
    return c;
}
// The same where both operands are contiguous in k: A(r, k) = pa[r sa + k],
// B(k, j) = pb[j sb + k] (rows 16-byte aligned, K a multiple of 16).  The
// sum over k is taken in another order: in block kb of 16, lane group
// kq = l / 16 supplies k = 16 kb + 4 kq + m to step m, so each lane reads
// its four k of A and of B with one 16-byte load each.
template <int K>
__device__ __forceinline__ f32x4 tile_mm_kc(const float *pa, int sa, const float *pb, int sb, f32x4 c, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    f32x4 av[K / 16], bv[K / 16];
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb) {
        av[kb] = *reinterpret_cast<const f32x4 *>(pa + r * sa + 16 * kb + 4 * kq);
        bv[kb] = *reinterpret_cast<const f32x4 *>(pb + r * sb + 16 * kb + 4 * kq);
    }
#pragma unroll
    for (int kb = 0; kb < K / 16; ++kb)
#pragma unroll
        for (int m = 0; m < 4; ++m) c = mfma4(av[kb][m], bv[kb][m], c);
    return c;
}

// the sum of x over the 16 lanes of each row, in every lane of the row
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp_mv<0xb1>(x);   // lane ^ 1
    x += dpp_mv<0x4e>(x);   // lane ^ 2
    x += dpp_mv<0x141>(x);  // the other quad of the 8
    x += dpp_mv<0x140>(x);  // the other 8 of the row
    return x;
}

// Forward substitution for one column of (I + A)^-1: lane (r, g) holds x_r of
// the column its row group solves, nar row r of -A.  At pivot u every row
// adds nar[u] times x_u, read from lane u of the same 16-lane row
// (row_newbcast); A is strictly lower triangular, so rows r <= u keep their
// value.
template <int U>
__device__ __forceinline__ void solve_pivots(float &x, const float (&nar)[16]) {
    if constexpr (U < 15) {
        x += nar[U] * dpp_mv<0x150 + U>(x);
        solve_pivots<U + 1>(x, nar);
    }
}

// Global accesses of the chunk kernel go through buffer descriptors: a
// wave-uniform base (token t0 of this (b, h)) with the number of bytes up to
// the end of the chunk's last valid token, plus a 32-bit offset per lane.
// Accesses of tokens past the end fall outside the range: loads return zeros
// and stores are dropped, so no lane needs a test or a branch (and the
// compiler can count the outstanding memory operations exactly).  The
// launcher keeps 16 H D 4 below 2^31.
using Rsrc = __amdgpu_buffer_rsrc_t;
using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Rsrc buf(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0), static_cast<int>(bytes),
                                            0x00020000);
}
__device__ __forceinline__ uint4 ld16(Rsrc r, uint32_t off) {
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ uint2 ld8(Rsrc r, uint32_t off) {
    const uint32_t __attribute__((ext_vector_type(2))) x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return make_uint2(x[0], x[1]);
}
__device__ __forceinline__ float4 ld16f(Rsrc r, uint32_t off) {
    const uint4 x = ld16(r, off);
    return make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
}
__device__ __forceinline__ void st4(Rsrc r, uint32_t off, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, off, 0, 0);
}
__device__ __forceinline__ void st16(Rsrc r, uint32_t off, f32x4 x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// A work-group barrier that orders LDS only: the waves' LDS writes are complete
// and visible after it, while their global loads (the next chunk's inputs)
// and stores (this chunk's outputs) stay in flight across it.  (A full
// barrier is a workgroup-scope fence, which on this target waits for every
// outstanding global access.)
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace
}  // namespace kda
