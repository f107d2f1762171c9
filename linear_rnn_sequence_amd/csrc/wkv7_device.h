// Device-side helpers shared by the WKV7 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkv7 {

// ---------------------------------------------------------------------------
// bf16 <-> f32.  Widening is exact (a 16-bit shift); narrowing rounds to
// nearest, ties to even, and keeps NaN a (quiet) NaN.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Four consecutive elements of a per-token vector, widened to float.
struct Bf16In {
    using elem = uint16_t;
    static __device__ __forceinline__ float4 load4(const uint16_t *p) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    static __device__ __forceinline__ void store4(uint16_t *p, float4 x) {
        uint2 u;
        u.x = pack_bf16x2(x.x, x.y);
        u.y = pack_bf16x2(x.z, x.w);
        *reinterpret_cast<uint2 *>(p) = u;
    }
    static __device__ __forceinline__ void store1(uint16_t *p, float x) {
        *p = (uint16_t)f32_to_bf16_rne(x);
    }
};

struct F32In {
    using elem = float;
    static __device__ __forceinline__ float4 load4(const float *p) {
        return *reinterpret_cast<const float4 *>(p);
    }
    static __device__ __forceinline__ void store4(float *p, float4 x) {
        *reinterpret_cast<float4 *>(p) = x;
    }
    static __device__ __forceinline__ void store1(float *p, float x) { *p = x; }
};

// Raw 4-element loads kept in flight in registers (prefetch), widened later.
template <class IO>
struct RawLoad;
template <>
struct RawLoad<Bf16In> {
    using T = uint2;
    static __device__ __forceinline__ T load(const void *p, long off) {
        return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p) + off);
    }
    static __device__ __forceinline__ float4 widen(T u) {
        return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
    }
    static __device__ __forceinline__ T zero() { return make_uint2(0u, 0u); }
};
template <>
struct RawLoad<F32In> {
    using T = float4;
    static __device__ __forceinline__ T load(const void *p, long off) {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(p) + off);
    }
    static __device__ __forceinline__ float4 widen(T u) { return u; }
    static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
};

// ---------------------------------------------------------------------------
// Cross-lane sums with DPP (no LDS traffic).  Lanes are grouped in DPP "rows"
// of 16; quad_perm swaps within groups of 4, row_half_mirror reverses each
// group of 8, row_mirror reverses the row of 16.  After the steps every lane
// of the group holds the group's sum.
// ---------------------------------------------------------------------------
constexpr int kDppQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowRor8 = 0x128;  // row_ror:8, lanes lo and lo ^ 8 of each row trade values

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ float sum_lanes8(float x) {
    x += dpp_mov<kDppQuadXor1>(x);
    x += dpp_mov<kDppQuadXor2>(x);
    x += dpp_mov<kDppRowHalfMirror>(x);
    return x;
}

__device__ __forceinline__ float sum_lanes16(float x) {
    x = sum_lanes8(x);
    x += dpp_mov<kDppRowMirror>(x);
    return x;
}

// Sum over the four DPP rows (lanes l, l^16, l^32, l^48), in VALU only:
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second, so with both operands x the two results add up to
// x + x^32 in every lane; v_permlane16_swap does the same between odd and even
// rows, giving + x^16.
__device__ __forceinline__ float sum_rows4(float x) {
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Four independent sums over the four DPP rows at the cost of three swaps:
// v_permlane32_swap pairs (a, b) so that lanes 0..31 add up a and lanes
// 32..63 add up b over lane bit 5 (likewise (c, d)); v_permlane16_swap then
// pairs the two results over lane bit 4.  Row 0 of the result holds the total
// of a, row 1 of c, row 2 of b, row 3 of d (see packed_col).
__device__ __forceinline__ float swap32_add(float a, float b) {
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                    false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}
__device__ __forceinline__ float swap16_add(float a, float b) {
    const auto h = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b),
                                                    false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}
__device__ __forceinline__ float sum_rows4_packed(float a, float b, float c, float d) {
    return swap16_add(swap32_add(a, b), swap32_add(c, d));
}
// Which of (a, b, c, d) = operands 0..3 the lanes of DPP row `row` hold.
__device__ __forceinline__ int packed_col(int row) { return (row & 1) * 2 + (row >> 1); }

}  // namespace wkv7
