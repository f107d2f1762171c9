// MFMA helpers shared by the chunked kernels (gfx950, wave64): operand types,
// the matrix-core opcodes with distinct accumulator types, bf16 conversion, and
// the unit lower-triangular inverse of a chunk.
//
// Lane layouts of v_mfma_f32_16x16x16_bf16 (lane l, g = l >> 4, lo = l & 15,
// e = 0..3):
//   A operand of P (16 x 16): lane holds P[lo][4g + e]
//   B operand of Q (16 x 16): lane holds Q[4g + e][lo]
//   result D(M):              lane holds M[4g + e][lo]
// so D(M) is the B operand of M and the A operand of M^T.  The 16x16x32 form
// holds 8 consecutive k per lane: with the two K = 16 operands of a pair side
// by side in the lanes (A0 | A1) and (B0 | B1), one instruction adds A0 B0 + A1 B1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef short bf16x8s __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Accumulator tile of the 16x16xK bf16 MFMA.  The two opcodes get distinct
// types so that the result of one cannot be passed as the accumulator of the
// other: a 16x16x16 result fed to a 16x16x32 a few instructions later was read
// stale.  Elements are read with [] and written through .v.
template <int K>
struct Acc {
    f32x4 v;
    __device__ __forceinline__ float operator[](int e) const { return v[e]; }
    static __device__ __forceinline__ Acc zero() { return Acc{f32x4{0.f, 0.f, 0.f, 0.f}}; }
};
using Acc16 = Acc<16>;
using Acc32 = Acc<32>;
using Acc4 = Acc<4>;  // v_mfma_f32_16x16x4_f32 (float32 operands)

__device__ __forceinline__ Acc16 mfma16(bf16x4 a, bf16x4 b, Acc16 c) {
    return Acc16{__builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c.v, 0, 0, 0)};
}
// c + A0 B0 + A1 B1 for a = (A0 | A1), b = (B0 | B1)
__device__ __forceinline__ Acc32 mfma32(bf16x8s a, bf16x8s b, Acc32 c) {
    return Acc32{__builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, b), c.v, 0,
                                                         0, 0)};
}

// float32 operands, K = 4: lane (g, lo) gives A[lo][k_g] and B[k_g][lo] for the
// instruction's g-th k.
__device__ __forceinline__ Acc4 mfma_f32(float a, float b, Acc4 c) {
    return Acc4{__builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c.v, 0, 0, 0)};
}

// k-block layout of a 16 x 16 M from its D layout: lane (g, lo) then holds
// M[4e + g][lo] at element e (a transpose of the 4 x 4 (row group, element)
// block of every column): v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second, v_permlane16_swap the odd
// rows of its first with the even rows of its second.
__device__ __forceinline__ f32x4 kblock(f32x4 x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[0]), __float_as_uint(x[2]),
                                                    false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[1]), __float_as_uint(x[3]),
                                                    false, false);
    const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
    const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
    return f32x4{__uint_as_float(c[0]), __uint_as_float(c[1]), __uint_as_float(d[0]),
                 __uint_as_float(d[1])};
}
// D(A B) in float32, summed over the k in the blocks of MASK (bit i: k = 4i ..
// 4i + 3; the others hold zeros of A or B), from ka = kblock(D(A^T)) and
// kb = kblock(D(B)): at element i lane (g, lo) holds A[lo][4i + g] and
// B[4i + g][lo], the operands of one v_mfma_f32_16x16x4_f32 for block i.
template <int MASK>
__device__ __forceinline__ f32x4 mul_kblocks(f32x4 ka, f32x4 kb) {
    Acc4 c = Acc4::zero();
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (MASK & (1 << i)) c = mfma_f32(ka[i], kb[i], c);
    return c.v;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32;
// written as a vector conversion so the compiler sees it and inserts the wait
// states an MFMA result needs before a VALU reads it)
__device__ __forceinline__ unsigned cvt_pk(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x4 to_bf16(f32x4 x) {
    const u32x2 v = {cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3])};
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ f32x4 from_bf16(bf16x4 b) {
    const u32x2 u = __builtin_bit_cast(u32x2, b);
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u),
                 __uint_as_float(u[1] << 16), __uint_as_float(u[1] & 0xffff0000u)};
}

// value of lane E of this lane's quad (DPP quad_perm [E, E, E, E])
template <int E>
__device__ __forceinline__ float quad_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), E * 0x55, 0xF, 0xF, true));
}

// X = (I + N)^-1 for a strictly lower-triangular 16 x 16 N (the coupling of a
// chunk's removal probes), given dn = D(N) and dnt = D(N^T) with every entry on
// or above the diagonal zero.  Returns dx = D(X) and dxt = D(X^T).
//
// Block substitution, whose intermediates never exceed the true inverse's
// blocks times N's (a product form such as (I - N)(I + N^2)(I + N^4)(I + N^8)
// builds up binomial-sized entries that must cancel, and fails for repeated or
// correlated removal keys), all in float32:
//  1. the four 4 x 4 diagonal blocks by forward substitution on the quad of
//     lanes that holds each block (column-wise for X, row-wise for X^T), the
//     entries of N broadcast within the quad;
//  2. for blocks of size 4, then 8: with N_l the entries of N below the
//     diagonal blocks of that size (t in the lower, s in the upper half of a
//     diagonal block of twice the size), T = N_l X and X <- X - X T (each new
//     block is -D^-1 C A^-1 from the diagonal blocks' inverses), and likewise
//     X^T <- X^T - T^T X^T, as float32 matrix-core products
//     (v_mfma_f32_16x16x4_f32, one per block of four k that is not all zero).
// A caller that uses only one of dx, dxt leaves the last level's other product
// to dead-code elimination.
__device__ __forceinline__ void tri_inverse(f32x4 dn, f32x4 dnt, int lane, f32x4 &dx,
                                            f32x4 &dxt) {
    const int g = lane >> 4, lo = lane & 15, e0 = lo & 3;
    const bool diag = (lo >> 2) == g;  // this quad holds diagonal block g
    // column lo of X's block: rows 4g + e; N[4g+e][4g+e'] is dn[e] of quad lane e'
    float x0 = e0 == 0 ? 1.f : 0.f;
    float x1 = (e0 == 1 ? 1.f : 0.f) - quad_bcast<0>(dn[1]) * x0;
    float x2 = (e0 == 2 ? 1.f : 0.f) - quad_bcast<0>(dn[2]) * x0 - quad_bcast<1>(dn[2]) * x1;
    float x3 = (e0 == 3 ? 1.f : 0.f) - quad_bcast<0>(dn[3]) * x0 - quad_bcast<1>(dn[3]) * x1 -
               quad_bcast<2>(dn[3]) * x2;
    // row lo of X's block (X^T's column): from X (I + N) = I, right to left;
    // N[4g+m][4g+s] is dnt[s] of quad lane m
    float y3 = e0 == 3 ? 1.f : 0.f;
    float y2 = (e0 == 2 ? 1.f : 0.f) - y3 * quad_bcast<3>(dnt[2]);
    float y1 = (e0 == 1 ? 1.f : 0.f) - y2 * quad_bcast<2>(dnt[1]) - y3 * quad_bcast<3>(dnt[1]);
    float y0 = (e0 == 0 ? 1.f : 0.f) - y1 * quad_bcast<1>(dnt[0]) - y2 * quad_bcast<2>(dnt[0]) -
               y3 * quad_bcast<3>(dnt[0]);
    dx = diag ? f32x4{x0, x1, x2, x3} : zero4();
    dxt = diag ? f32x4{y0, y1, y2, y3} : zero4();
    // N in k-block layout: element i of lane (g, lo) is N[t = lo][s = 4i + g]
    const f32x4 kn = kblock(dnt);
    f32x4 n4, n8;  // N below the diagonal blocks of size 4, and of size 8
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        n4[i] = ((lo >> 3) == (i >> 1) && ((lo >> 2) & 1) && !(i & 1)) ? kn[i] : 0.f;
        n8[i] = (lo >= 8 && i < 2) ? kn[i] : 0.f;
    }
    {  // blocks of size 4: N_4 has columns in k-blocks 0, 2 and T its rows in 1, 3
        const f32x4 kx = kblock(dx), kxt = kblock(dxt);
        const f32x4 kt = kblock(mul_kblocks<0x5>(n4, kx));  // T = N_4 X
        dx = dx - mul_kblocks<0xA>(kxt, kt);                // X - X T
        dxt = dxt - mul_kblocks<0xA>(kt, kxt);              // X^T - T^T X^T
    }
    {  // blocks of size 8: N_8 has columns in k-blocks 0, 1 and T its rows in 2, 3
        const f32x4 kx = kblock(dx), kxt = kblock(dxt);
        const f32x4 kt = kblock(mul_kblocks<0x3>(n8, kx));
        dx = dx - mul_kblocks<0xC>(kxt, kt);
        dxt = dxt - mul_kblocks<0xC>(kt, kxt);
    }
}

}  // namespace wkv7
