// WKV7 single-token step over a batch of resident states (decode).
//
// One token of the recurrence (RWKV-7 "Goose" author response, numpy
// time_mixing listing) for each of B*H heads whose float32 states live in HBM:
//   u_i = sum_j S_ij kappa_j
//   S_ij <- S_ij w_j - u_i (a_j kappa_j) + v_i k_j      (written back in place)
//   y_i = sum_j S_ij (w_j r_j) + v_i (k . r) - u_i ((a*kappa) . r)  (= S_new r)
// This is the constant-memory single-token inference of the RWKV-7 "Goose"
// summary, §8 Speed and Memory.  The state read and write (32 KiB per head)
// is all but the whole traffic, so the kernel is laid out for HBM streaming.
//
// One workgroup per head, 4 value rows per lane: at head size 64 four waves of
// 16 rows (256 threads), at 128 sixteen waves of 8 rows (1024 threads, 32
// lanes per row; see DecodeShape).  The GroupNorm statistics of the fused
// epilogue meet in LDS.  (Measured against 1, 2, 4, 8 and 16 value rows per
// lane, one wave per workgroup, one, two and four heads per workgroup, and
// persistent waves: this layout streamed fastest, ~80% of 8 TB/s at head size
// 64, level with the best plain copy kernel found at the same launch size.
// Workgroups of a single wave were held back by the rate at which workgroups
// are dispatched.)
// Lane (c, g) = (lane & 15, lane >> 4) owns key columns 4c .. 4c+3 of value
// rows r0 + 4g .. r0 + 4g + 3: every state load instruction reads four complete
// 256-byte rows (16 lanes x 16 bytes each; at head size 128, two 512-byte
// rows), so each wave moves its 4 KiB in four fully coalesced dwordx4 loads
// issued back to back.  Row sums (S kappa and S (w*r)) are DPP reductions over
// a row's lanes.  Lanes c < 4 finally hold y of rows r0 + 4g + c, so each
// wave's readouts leave as one contiguous store.
// State loads and stores are non-temporal: each state is touched once per call
// and the next layer's states should not be evicted for it.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ f32x4 ld_state(const float *p) {
    if (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
    return *reinterpret_cast<const f32x4 *>(p);
}
template <bool NT>
__device__ __forceinline__ void st_state(float *p, f32x4 x) {
    if (NT)
        __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
    else
        *reinterpret_cast<f32x4 *>(p) = x;
}

// R consecutive elements (value rows r .. r+R-1, R = 4 or 8), widened to float.
template <int R>
__device__ __forceinline__ void load_rows(const uint16_t *p, float *out) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
        const uint2 a = *reinterpret_cast<const uint2 *>(p + 4 * q);
        out[4 * q] = bf16_lo(a.x); out[4 * q + 1] = bf16_hi(a.x);
        out[4 * q + 2] = bf16_lo(a.y); out[4 * q + 3] = bf16_hi(a.y);
    }
}
template <int R>
__device__ __forceinline__ void load_rows(const float *p, float *out) {
#pragma unroll
    for (int q = 0; q < R / 4; ++q) {
        const float4 x = *reinterpret_cast<const float4 *>(p + 4 * q);
        out[4 * q] = x.x; out[4 * q + 1] = x.y; out[4 * q + 2] = x.z; out[4 * q + 3] = x.w;
    }
}

// Lane layout for head size N: N/4 lanes cover one state row (4 key columns
// each, 16 bytes), so a wave holds 64/(N/4) row groups of kRows rows.
template <int N>
struct DecodeShape {
    static constexpr int kRows = 4;                             // value rows per lane
    static constexpr int kLanesPerRow = N / 4;                  // 16 (N=64) or 32 (N=128)
    static constexpr int kGroups = 64 / kLanesPerRow;           // 4 or 2
    static constexpr int kRowsPerWave = kGroups * kRows;        // 16 or 8
    static constexpr int kWavesPerHead = N / kRowsPerWave;      // 4 or 16: one workgroup
};

// Sum over the lanes of one state row (16 or 32 lanes).
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    x = sum_lanes16(x);
    if constexpr (N == 128) x = swap16_add(x, x);  // adjacent DPP rows: lanes l, l^16
    return x;
}

template <class IO, bool EPI, bool NT, bool W32, int N, bool FUSED = false>
__global__ __launch_bounds__(64 * DecodeShape<N>::kWavesPerHead) void decode_kernel(
    DecodeArgs p) {
    using E = typename IO::elem;
    using Sh = DecodeShape<N>;
    constexpr int kW = Sh::kWavesPerHead;
    constexpr int kRows = Sh::kRows;
    __shared__ float2 xch[kW];  // epilogue: (mean, M2) of each wave's rows
    const int lane = threadIdx.x & 63;
    const long head = (long)blockIdx.x;
    const int part = (int)(threadIdx.x >> 6);
    if (head >= (long)p.B * p.H) return;  // whole workgroup leaves together
    const int h = (int)(head % p.H);
    const int c = lane % Sh::kLanesPerRow, g = lane / Sh::kLanesPerRow;
    const int r0 = Sh::kRowsPerWave * part + kRows * g;  // this lane's value rows r0 .. +kRows-1

    float *st = p.state + head * (N * N) + r0 * N + 4 * c;
    f32x4 S[kRows];
#pragma unroll
    for (int m = 0; m < kRows; ++m) S[m] = ld_state<NT>(st + m * N);

    const long vo = head * N;
    const E *pr = static_cast<const E *>(p.r) + vo;
    const float4 w = W32 ? F32In::load4(static_cast<const float *>(p.w) + vo + 4 * c)
                         : IO::load4(static_cast<const E *>(p.w) + vo + 4 * c);
    const float4 a = IO::load4(static_cast<const E *>(p.a) + vo + 4 * c);
    float4 k = IO::load4(static_cast<const E *>(p.k) + vo + 4 * c);
    float4 kap;
    if (FUSED) {
        // time-mix prologue from raw keys: kappa = normalise(k * k_k) over the
        // head's N channels (this row's lanes), k <- k + k (a-1) k_a
        const float4 kk4 = *reinterpret_cast<const float4 *>(p.k_k + h * N + 4 * c);
        const float4 ka4 = *reinterpret_cast<const float4 *>(p.k_a + h * N + 4 * c);
        const float4 kk = make_float4(k.x * kk4.x, k.y * kk4.y, k.z * kk4.z, k.w * kk4.w);
        const float ss = row_sum<N>(kk.x * kk.x + kk.y * kk.y + kk.z * kk.z + kk.w * kk.w);
        const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
        kap = make_float4(kk.x * inv, kk.y * inv, kk.z * inv, kk.w * inv);
        k = make_float4(k.x + k.x * (a.x - 1.f) * ka4.x, k.y + k.y * (a.y - 1.f) * ka4.y,
                        k.z + k.z * (a.z - 1.f) * ka4.z, k.w + k.w * (a.w - 1.f) * ka4.w);
    } else {
        kap = IO::load4(static_cast<const E *>(p.kappa) + vo + 4 * c);
    }
    const float4 r = IO::load4(pr + 4 * c);
    float v[kRows];
    load_rows<kRows>(static_cast<const E *>(p.v) + vo + r0, v);

    const float4 bb = make_float4(a.x * kap.x, a.y * kap.y, a.z * kap.z, a.w * kap.w);
    const float4 wr = make_float4(w.x * r.x, w.y * r.y, w.z * r.z, w.w * r.w);
    float kr = k.x * r.x + k.y * r.y + k.z * r.z + k.w * r.w;
    float br = bb.x * r.x + bb.y * r.y + bb.z * r.z + bb.w * r.w;
    float bon = 0.f;
    if (EPI) {
        const float4 rk = *reinterpret_cast<const float4 *>(p.epi.r_k + h * N + 4 * c);
        bon = r.x * k.x * rk.x + r.y * k.y * rk.y + r.z * k.z * rk.z + r.w * k.w * rk.w;
    }

    float u[kRows], y[kRows];
#pragma unroll
    for (int m = 0; m < kRows; ++m) {
        u[m] = S[m].x * kap.x + S[m].y * kap.y + S[m].z * kap.z + S[m].w * kap.w;
        y[m] = S[m].x * wr.x + S[m].y * wr.y + S[m].z * wr.z + S[m].w * wr.w;
    }
#pragma unroll
    for (int m = 0; m < kRows; ++m) {
        u[m] = row_sum<N>(u[m]);
        y[m] = row_sum<N>(y[m]);
    }
    kr = row_sum<N>(kr);
    br = row_sum<N>(br);
    if (EPI) bon = row_sum<N>(bon);

#pragma unroll
    for (int m = 0; m < kRows; ++m) {
        y[m] = y[m] + v[m] * kr - u[m] * br;
        f32x4 s = S[m];
        s.x = s.x * w.x - u[m] * bb.x + v[m] * k.x;
        s.y = s.y * w.y - u[m] * bb.y + v[m] * k.y;
        s.z = s.z * w.z - u[m] * bb.z + v[m] * k.z;
        s.w = s.w * w.w - u[m] * bb.w + v[m] * k.w;
        st_state<NT>(st + m * N, s);
    }

    // lane c < kRows keeps row r0 + c
    const int sel = c & (kRows - 1);
    float yo = y[0], vo1 = v[0];
#pragma unroll
    for (int m = 1; m < kRows; ++m) {
        yo = (sel == m) ? y[m] : yo;
        vo1 = (sel == m) ? v[m] : vo1;
    }
    if (EPI) {
        // statistics of this wave's rows, then Chan's combination over the head's waves
        float s1 = 0.f;
#pragma unroll
        for (int m = 0; m < kRows; ++m) s1 += y[m];
        // sum over the wave's row groups (every lane of a group holds its rows' sums)
        s1 = (N == 64) ? sum_rows4(s1) : swap32_add(s1, s1);
        const float mu_w = s1 * (1.f / Sh::kRowsPerWave);
        float s2 = 0.f;
#pragma unroll
        for (int m = 0; m < kRows; ++m) s2 += (y[m] - mu_w) * (y[m] - mu_w);
        const float m2_w = (N == 64) ? sum_rows4(s2) : swap32_add(s2, s2);
        if (lane == 0) xch[part] = make_float2(mu_w, m2_w);
        __syncthreads();
        float mu = 0.f;
#pragma unroll
        for (int q = 0; q < kW; ++q) mu += xch[q].x;
        mu *= 1.f / kW;
        float m2 = 0.f, dev = 0.f;
#pragma unroll
        for (int q = 0; q < kW; ++q) {
            const float2 x = xch[q];
            m2 += x.y;
            dev += (x.x - mu) * (x.x - mu);
        }
        const float var = (m2 + (float)Sh::kRowsPerWave * dev) * (1.f / N);
        const float rs = __builtin_amdgcn_rsqf(var + p.epi.eps);
        const int ch = h * N + r0 + sel;
        const float gw = p.epi.ln_w ? p.epi.ln_w[ch] : 1.f;
        const float gb = p.epi.ln_b ? p.epi.ln_b[ch] : 0.f;
        yo = (yo - mu) * rs * gw + gb + bon * vo1;
    }
    if (FUSED && p.g) {  // output gate
        float gv[kRows];
        load_rows<kRows>(static_cast<const E *>(p.g) + vo + r0, gv);
        float gsel = gv[0];
#pragma unroll
        for (int m = 1; m < kRows; ++m) gsel = (sel == m) ? gv[m] : gsel;
        yo *= gsel;
    }
    if (c < kRows) IO::store1(static_cast<E *>(p.y) + vo + r0 + c, yo);
}

template <int N, class IO, bool W32, bool FUSED>
hipError_t launch_decode_n(const DecodeArgs &p, hipStream_t stream) {
    constexpr int kW = DecodeShape<N>::kWavesPerHead;
    const long heads = (long)p.B * p.H;
    // one workgroup per head holding all its waves
    if (p.epilogue)
        hipLaunchKernelGGL((decode_kernel<IO, true, true, W32, N, FUSED>), dim3((unsigned)heads),
                           dim3(64 * kW), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<IO, false, true, W32, N, FUSED>), dim3((unsigned)heads),
                           dim3(64 * kW), 0, stream, p);
    return hipGetLastError();
}

template <int N>
hipError_t launch_decode_dt(const DecodeArgs &p, hipStream_t stream) {
    if (p.fused)  // (the fused prologue comes with one dtype for all vectors)
        return p.bf16 ? launch_decode_n<N, Bf16In, false, true>(p, stream)
                      : launch_decode_n<N, F32In, false, true>(p, stream);
    if (p.bf16 && p.w32) return launch_decode_n<N, Bf16In, true, false>(p, stream);
    if (p.bf16) return launch_decode_n<N, Bf16In, false, false>(p, stream);
    return launch_decode_n<N, F32In, false, false>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs &p, hipStream_t stream) {
    return p.N == 128 ? launch_decode_dt<128>(p, stream) : launch_decode_dt<64>(p, stream);
}

}  // namespace wkv7
