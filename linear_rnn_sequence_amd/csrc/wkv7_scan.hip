// WKV7 sequential scan (ALGO_SCAN): the recurrence token by token, with each
// head's N x N float32 state (N = 64 or 128) held in VGPRs for the whole
// sequence.
//
// Per token (RWKV-7 "Goose" author response, numpy time_mixing listing; the
// ARWKV verdict's key_machinery field gives the same update in row form):
//   u_i = sum_j S_ij kappa_j                        (old state)
//   S_ij <- S_ij w_j - u_i (a_j kappa_j) + v_i k_j
//   y_i = sum_j S_ij r_j                            (new state)
// The readout is evaluated from the old state in the same pass as u, using
//   y_i = sum_j S_ij (w_j r_j) + v_i (k . r) - u_i ((a*kappa) . r),
// which is the same sum regrouped, so one cross-lane reduction serves both.
//
// Work split.  One workgroup (N/16 waves) per (batch, head).  Value rows are
// independent (row i of S only ever meets v_i and u_i), so wave w owns rows
// 16w .. 16w+15; inside a wave a lane owns 2 rows x N/8 key columns and the
// row sums need an 8-lane DPP reduction.  The per-token vectors are staged
// 16 tokens at a time: every thread widens one 4-column slice of one token
// (bf16 -> f32 is exact), forms a*kappa, w*r and the per-token scalars
// k.r, (a*kappa).r and the bonus sum, and writes them to LDS; the loads of the
// next 16 tokens are in flight while the current ones are consumed.  The
// readouts of the 16 tokens are gathered in LDS and written out coalesced
// (with the optional GroupNorm + bonus epilogue applied on the way).
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int kTC = 16;  // tokens staged per round

template <int N>
struct ScanShape {
    static constexpr int kThreads = 4 * N;   // N/16 waves of 16 rows
    static constexpr int kCols = N / 8;      // key columns per lane (8 lanes per row)
    static constexpr int kStage = N / 4;     // staging lanes per token (4 channels each)
};

template <int N>
struct __align__(16) ScanStage {
    float kap[kTC][N];
    float w[kTC][N];
    float b[kTC][N];   // a * kappa
    float k[kTC][N];
    float wr[kTC][N];  // w * r
    float v[kTC][N];
    float4 sc[kTC];    // x = k.r, y = (a*kappa).r, z = sum_j r_j k_j r_k[j]
    float ybuf[kTC][N];
};

// Sum over the staging lanes of one token (16 lanes for N = 64, 32 for 128).
template <int N>
__device__ __forceinline__ float stage_sum(float x) {
    x = sum_lanes16(x);
    if constexpr (N == 128) x = swap16_add(x, x);
    return x;
}

__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ __forceinline__ float4 mul4(float4 a, float4 b) {
    return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}

template <bool W32, class L>
struct DecayLoad {
    using type = L;
};
template <class L>
struct DecayLoad<true, L> {
    using type = RawLoad<F32In>;  // w as float32
};

template <class IO, bool EPI, bool W32, int N>
__global__ __launch_bounds__(ScanShape<N>::kThreads) void scan_kernel(ForwardArgs p) {
    using L = RawLoad<IO>;
    using LW = typename DecayLoad<W32, L>::type;
    using E = typename IO::elem;
    constexpr int kCols = ScanShape<N>::kCols;
    __shared__ ScanStage<N> st;

    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = p.T;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int c = lane & 7, g = lane >> 3;
    const int i0 = wave * 16 + 2 * g;  // value rows i0, i0 + 1
    const int j0 = kCols * c;          // key columns j0 .. j0 + kCols - 1
    // elements from one token to the next in processing order (negative when the
    // sequence is walked from its end) and the offset of the first processed token
    const long HN = p.reverse ? -(long)p.H * N : (long)p.H * N;
    const long tok0 = ((long)b * T + (p.reverse ? T - 1 : 0)) * ((long)p.H * N) + (long)h * N;
    // staging role: token, 4-column slice
    const int s_t = tid / ScanShape<N>::kStage, s_q = tid % ScanShape<N>::kStage;

    // the lane's state columns moved as float4s
    auto ld_rows = [&](const float *base, float (&S)[2][kCols]) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int q = 0; q < kCols / 4; ++q) {
                const float4 x = *reinterpret_cast<const float4 *>(base + (i0 + r) * N + j0 + 4 * q);
                S[r][4 * q] = x.x; S[r][4 * q + 1] = x.y; S[r][4 * q + 2] = x.z; S[r][4 * q + 3] = x.w;
            }
    };
    auto st_rows = [&](float *base, const float (&S)[2][kCols]) {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int q = 0; q < kCols / 4; ++q)
                *reinterpret_cast<float4 *>(base + (i0 + r) * N + j0 + 4 * q) =
                    make_float4(S[r][4 * q], S[r][4 * q + 1], S[r][4 * q + 2], S[r][4 * q + 3]);
    };

    float S[2][kCols];
    const long sb = (long)bh * N * N;
    if (p.s0) {
        ld_rows(p.s0 + sb, S);
    } else {
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int e = 0; e < kCols; ++e) S[r][e] = 0.f;
    }

    // fused prologue parameters of this staging thread's 4 channels
    float4 kk4p = make_float4(0.f, 0.f, 0.f, 0.f), ka4p = kk4p;
    if (p.fused) {
        kk4p = *reinterpret_cast<const float4 *>(p.k_k + h * N + 4 * s_q);
        ka4p = *reinterpret_cast<const float4 *>(p.k_a + h * N + 4 * s_q);
    }
    float4 rk4 = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 lnw4 = make_float4(1.f, 1.f, 1.f, 1.f), lnb4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (EPI) {
        rk4 = *reinterpret_cast<const float4 *>(p.epi.r_k + h * N + 4 * s_q);
        if (p.epi.ln_w) lnw4 = *reinterpret_cast<const float4 *>(p.epi.ln_w + h * N + 4 * s_q);
        if (p.epi.ln_b) lnb4 = *reinterpret_cast<const float4 *>(p.epi.ln_b + h * N + 4 * s_q);
    }

    typename L::T xr, xk, xv, xkap, xa;
    typename LW::T xw;
    // the loads of a round, without a branch around them (one that assigns the
    // registers on two paths keeps them in scratch memory): a token past T
    // reads token T-1 and is zeroed at use
    bool x_ok = false;
    auto issue = [&](int chunk) {
        const int t = chunk * kTC + s_t;
        x_ok = t < T;
        const long off = tok0 + (long)min(t, T - 1) * HN + 4 * s_q;
        xr = L::load(p.r, off);
        xw = LW::load(p.w, off);
        xk = L::load(p.k, off);
        xv = L::load(p.v, off);
        xkap = L::load(p.fused ? p.k : p.kappa, off);  // (unused when fused)
        xa = L::load(p.a, off);
    };

    const int nchunks = (T + kTC - 1) / kTC;
    static_assert(kTC == kCkpt, "a staging round is one checkpoint interval");
    issue(0);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int tl = min(kTC, T - ch * kTC);
        if (p.s_ckpt)  // the state before token ch * kTC
            st_rows(p.s_ckpt + ((long)bh * nchunks + ch) * N * N, S);
        // ---- stage this chunk's vectors ----
        const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 r4 = x_ok ? L::widen(xr) : z4, w4 = x_ok ? LW::widen(xw) : z4;
        float4 k4 = x_ok ? L::widen(xk) : z4, kap4 = x_ok ? L::widen(xkap) : z4;
        const float4 v4 = x_ok ? L::widen(xv) : z4, a4 = x_ok ? L::widen(xa) : z4;
        if (p.fused) {
            // kappa = normalise(k * k_k) over the token's N channels (its staging
            // lanes); k <- k + k (a-1) k_a
            const float4 kk = mul4(k4, kk4p);
            const float inv = 1.f / fmaxf(sqrtf(stage_sum<N>(dot4(kk, kk))), 1e-12f);
            kap4 = make_float4(kk.x * inv, kk.y * inv, kk.z * inv, kk.w * inv);
            k4 = make_float4(k4.x + k4.x * (a4.x - 1.f) * ka4p.x, k4.y + k4.y * (a4.y - 1.f) * ka4p.y,
                             k4.z + k4.z * (a4.z - 1.f) * ka4p.z, k4.w + k4.w * (a4.w - 1.f) * ka4p.w);
        }
        const float4 b4 = mul4(a4, kap4);
        const float4 wr4 = mul4(w4, r4);
        float kr = stage_sum<N>(dot4(k4, r4));
        float br = stage_sum<N>(dot4(b4, r4));
        float bon = 0.f;
        if (EPI) bon = stage_sum<N>(dot4(mul4(r4, k4), rk4));
        __syncthreads();  // the previous round is done with the staging area
        *reinterpret_cast<float4 *>(&st.kap[s_t][4 * s_q]) = kap4;
        *reinterpret_cast<float4 *>(&st.w[s_t][4 * s_q]) = w4;
        *reinterpret_cast<float4 *>(&st.b[s_t][4 * s_q]) = b4;
        *reinterpret_cast<float4 *>(&st.k[s_t][4 * s_q]) = k4;
        *reinterpret_cast<float4 *>(&st.wr[s_t][4 * s_q]) = wr4;
        *reinterpret_cast<float4 *>(&st.v[s_t][4 * s_q]) = v4;
        if (s_q == 0) st.sc[s_t] = make_float4(kr, br, bon, 0.f);
        __syncthreads();
        if (ch + 1 < nchunks) issue(ch + 1);

        // ---- the recurrence over this chunk's tokens ----
        // a token's columns are read from LDS one token ahead, alternating
        // between two register sets, so the reads overlap the previous token
        struct Cols {
            float kap[kCols], w[kCols], bb[kCols], kk[kCols], wr[kCols];
            float2 vv;
            float4 sc;
        };
        auto ld_tok = [&](Cols &d, int tt) {
            auto ld_cols = [&](const float (&arr)[kTC][N], float (&dst)[kCols]) {
#pragma unroll
                for (int q = 0; q < kCols / 4; ++q) {
                    const float4 x = *reinterpret_cast<const float4 *>(&arr[tt][j0 + 4 * q]);
                    dst[4 * q] = x.x; dst[4 * q + 1] = x.y; dst[4 * q + 2] = x.z; dst[4 * q + 3] = x.w;
                }
            };
            ld_cols(st.kap, d.kap);
            ld_cols(st.w, d.w);
            ld_cols(st.b, d.bb);
            ld_cols(st.k, d.kk);
            ld_cols(st.wr, d.wr);
            d.vv = *reinterpret_cast<const float2 *>(&st.v[tt][i0]);
            d.sc = st.sc[tt];
        };
        auto step = [&](const Cols &x, int tt) {
            float pu0 = 0.f, pu1 = 0.f, py0 = 0.f, py1 = 0.f;
#pragma unroll
            for (int e = 0; e < kCols; ++e) {
                pu0 += S[0][e] * x.kap[e];
                pu1 += S[1][e] * x.kap[e];
                py0 += S[0][e] * x.wr[e];
                py1 += S[1][e] * x.wr[e];
            }
            pu0 = sum_lanes8(pu0);
            pu1 = sum_lanes8(pu1);
            py0 = sum_lanes8(py0);
            py1 = sum_lanes8(py1);
            const float y0 = py0 + x.vv.x * x.sc.x - pu0 * x.sc.y;
            const float y1 = py1 + x.vv.y * x.sc.x - pu1 * x.sc.y;
#pragma unroll
            for (int e = 0; e < kCols; ++e) {
                S[0][e] = S[0][e] * x.w[e] - pu0 * x.bb[e] + x.vv.x * x.kk[e];
                S[1][e] = S[1][e] * x.w[e] - pu1 * x.bb[e] + x.vv.y * x.kk[e];
            }
            if (c == 0) *reinterpret_cast<float2 *>(&st.ybuf[tt][i0]) = make_float2(y0, y1);
        };
        if constexpr (N == 64) {
            Cols ca, cb;
            ld_tok(ca, 0);
            for (int tt = 0; tt < tl; tt += 2) {
                ld_tok(cb, min(tt + 1, kTC - 1));
                step(ca, tt);
                if (tt + 1 < tl) {
                    ld_tok(ca, min(tt + 2, kTC - 1));
                    step(cb, tt + 1);
                }
            }
        } else {  // N = 128: two sets of 16 columns would not fit in registers
            for (int tt = 0; tt < tl; ++tt) {
                Cols cx;
                ld_tok(cx, tt);
                step(cx, tt);
            }
        }
        __syncthreads();

        // ---- readouts of this chunk: epilogue and coalesced store ----
        // (s_t is uniform over each token's staging lanes, so the reductions
        // below see all of their lanes active)
        if (s_t < tl) {
            const int t = ch * kTC + s_t;
            const long yo = tok0 + (long)t * HN + 4 * s_q;
            float4 y4 = *reinterpret_cast<const float4 *>(&st.ybuf[s_t][4 * s_q]);
            if (p.y_add) {  // the other direction's readouts
                const float4 ya = *reinterpret_cast<const float4 *>(p.y_add + yo);
                y4.x += ya.x; y4.y += ya.y; y4.z += ya.z; y4.w += ya.w;
            }
            if (EPI) {
                const float mu = stage_sum<N>(y4.x + y4.y + y4.z + y4.w) * (1.f / N);
                const float4 d = make_float4(y4.x - mu, y4.y - mu, y4.z - mu, y4.w - mu);
                const float var = stage_sum<N>(dot4(d, d)) * (1.f / N);
                const float rs = 1.f / sqrtf(var + p.epi.eps);
                const float bz = st.sc[s_t].z;
                const float4 vz = *reinterpret_cast<const float4 *>(&st.v[s_t][4 * s_q]);
                y4.x = d.x * rs * lnw4.x + lnb4.x + bz * vz.x;
                y4.y = d.y * rs * lnw4.y + lnb4.y + bz * vz.y;
                y4.z = d.z * rs * lnw4.z + lnb4.z + bz * vz.z;
                y4.w = d.w * rs * lnw4.w + lnb4.w + bz * vz.w;
            }
            if (p.g) {  // output gate (fused prologue)
                const float4 g4 = L::widen(L::load(p.g, yo));
                y4.x *= g4.x; y4.y *= g4.y; y4.z *= g4.z; y4.w *= g4.w;
            }
            if (p.y_f32)  // float32 readouts (first pass of a bidirectional call)
                *reinterpret_cast<float4 *>(p.y_f32 + yo) = y4;
            else
                IO::store4(static_cast<E *>(p.y) + yo, y4);
        }
    }

    if (p.s_out) st_rows(p.s_out + sb, S);
}

}  // namespace

namespace {

template <int N>
hipError_t launch_scan_n(const ForwardArgs &p, hipStream_t stream) {
    const dim3 grid((unsigned)((long)p.B * p.H)), block(ScanShape<N>::kThreads);
    if (p.bf16 && p.w32) {
        if (p.epilogue)
            hipLaunchKernelGGL((scan_kernel<Bf16In, true, true, N>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((scan_kernel<Bf16In, false, true, N>), grid, block, 0, stream, p);
    } else if (p.bf16) {
        if (p.epilogue)
            hipLaunchKernelGGL((scan_kernel<Bf16In, true, false, N>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((scan_kernel<Bf16In, false, false, N>), grid, block, 0, stream, p);
    } else {
        if (p.epilogue)
            hipLaunchKernelGGL((scan_kernel<F32In, true, false, N>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((scan_kernel<F32In, false, false, N>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_scan(const ForwardArgs &p, hipStream_t stream) {
    return p.N == 128 ? launch_scan_n<128>(p, stream) : launch_scan_n<64>(p, stream);
}

}  // namespace wkv7
