// WKV7 backward pass: gradients of L = sum_t <y_t, dy_t> + <S_T, dS_T> for the
// bare recurrence (RWKV-7 "Goose" author response, numpy time_mixing listing;
// ARWKV verdict, key_machinery field, row form)
//   u_t = S_{t-1} kappa_t,  b_t = a_t * kappa_t
//   S_t = S_{t-1} diag(w_t) - u_t b_t^T + v_t k_t^T,  y_t = S_t r_t
// walked in reverse.  With G the cotangent of S_t (G = dS_T at t = T-1, plus
// dy_t r_t^T):
//   dr_t = S_t^T dy_t          dv_t = G k_t          dk_t = G^T v_t
//   dw_t[j] = sum_i G_ij S_{t-1,ij}                  db_t = -G^T u_t
//   du_t = -G b_t              dkappa_t = S_{t-1}^T du_t + a_t * db_t
//   da_t = kappa_t * db_t      cotangent of S_{t-1} = G diag(w_t) + du_t kappa_t^T
// The training forward stored S before every 16th token; each interval's
// per-token states are recomputed from that state in fp32.
//
// Work split.  Value rows are independent in both directions (row i of S and
// of G only meets v_i, u_i, dy_i, du_i), so a workgroup of 4 waves owns a band
// of value rows and every key column, and lane (rg, cg) holds four rows and key
// columns 4cg .. 4cg+3 of S, of the recomputed states and of G (16 floats of
// each, whatever the head size):
//   N = 64:  one workgroup per (batch, head); wave w owns rows 16w .. 16w+15,
//            four row groups of 16 lanes;
//   N = 128: four workgroups per (batch, head), 32 rows each; wave w owns 8
//            rows, two row groups of 32 lanes.
// Row sums (u, dv, du) are DPP reductions over a row group's lanes; the column
// sums (dr, dk, db, dw and the S^T du part of dkappa) are outputs only, so they
// are reduced over the wave's row groups with permlane swaps and left per wave
// in LDS, and the four waves' parts are added when a block of tokens is written
// out.  At N = 64 that is the whole sum and the gradients are written directly.
// At N = 128 each workgroup writes its partial column sums (float32) to the
// workspace, and a second kernel adds the four parts in a fixed order and forms
// dr, dk, dw, dkappa = S^T du + a db and da = kappa db.  To bound that
// workspace the sequence is cut into slices walked last to first, each slice's
// cotangent of its entry state carried to the next launch in the workspace
// (each lane reads and writes only its own rows).
//
// Per 16-token interval, in reverse: the interval's inputs and dy are staged
// in LDS as fp32 (the previous interval's loads are in flight meanwhile); then
// for each 4-token block, last first, the states before its tokens are
// recomputed from the interval's stored state, kept in registers, and the four
// tokens are walked backwards.  Padding tokens past T carry w = 1 and zeros
// elsewhere, which leaves S and G unchanged.
#include <type_traits>

#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBlk = 4;                // tokens per recompute block
constexpr int kNBlk = kCkpt / kBlk;    // blocks per interval
constexpr int kNCol = 5;               // column sums: dr, dk, db, dw, S^T du
constexpr int kCombineThreads = 256;

// Lane and workgroup geometry at head size N (four waves per workgroup).
template <int N>
struct BwdGeo {
    static constexpr int RG = 256 / N;   // row groups per wave
    static constexpr int LR = N / 4;     // lanes per row group (four key columns each)
    static constexpr int RW = 4 * RG;    // value rows per wave
    static constexpr int RB = 4 * RW;    // value rows per workgroup
    static constexpr int P = N / RB;     // workgroups per head
    static constexpr int SLOTS = kCkpt * LR / kBwdThreads;  // staging slots per thread
    static_assert(P * RB == N && SLOTS * kBwdThreads == kCkpt * LR, "geometry");
};

// LDS.  At N = 128 (partial sums) the column sums leave after every token
// instead of every block of kBlk tokens, a is not staged (the second kernel
// forms dkappa and da) and v, dy only for the band's rows: 65 KB, so two
// workgroups share a CU.
template <int N>
struct __align__(16) BwdSmem {
    using Geo = BwdGeo<N>;
    static constexpr int CT = Geo::P > 1 ? 1 : kBlk;  // tokens per write-out
    float r[kCkpt][N], w[kCkpt][N], k[kCkpt][N], v[kCkpt][Geo::RB];
    float kap[kCkpt][N], a[kCkpt][Geo::P > 1 ? 4 : N], b[kCkpt][N], dy[kCkpt][Geo::RB];
    float col[2][4][CT][kNCol][N];  // [buffer][wave][token][sum][column]
    float dv[2][CT][Geo::RB];       // [buffer][token][row of the band]
};

// One slice of the sequence: intervals [c_begin, c_end) of kCkpt tokens.
struct BwdSlice {
    int c_begin, c_end;
    const float *g_in;  // cotangent of the state after the slice, or nullptr (zero)
    float *g_out;       // cotangent of the state before it, or nullptr (not written)
    float *part;        // N = 128: partial column sums [kNCol][P][B][L][H][N]
    int L;              // tokens per slice held by `part`
};

__device__ __forceinline__ float4 lds4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

// Sum over the lanes of a row group (16 lanes at N = 64, 32 at N = 128).
template <int N>
__device__ __forceinline__ float row_sum(float x) {
    x = sum_lanes16(x);
    if constexpr (N == 128) x = swap16_add(x, x);
    return x;
}

// At N = 128 with bf16 vectors two workgroups share a CU (LDS 65 KB each, at
// most 256 registers per lane; the compiler spills a few): measured on the
// 2.9B width (B8 T4096 H20), 15.4 ms against 21.1 ms with one.  The float32
// variant would spill about 90 registers and keeps one.
template <class IO, int N>
constexpr int kBwdWavesPerEU = (N == 128 && std::is_same<IO, Bf16In>::value) ? 2 : 1;

template <class IO, bool W32, int N>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(
    kBwdWavesPerEU<IO, N>))) void backward_kernel(BackwardArgs p, BwdSlice sl) {
    using Geo = BwdGeo<N>;
    using L = RawLoad<IO>;
    using LW = std::conditional_t<W32, RawLoad<F32In>, L>;  // the decay's loads
    using IOW = std::conditional_t<W32, F32In, IO>;         // the decay gradient's stores
    using E = typename IO::elem;
    using EW = typename IOW::elem;
    constexpr bool kPart = Geo::P > 1;  // partial column sums to the workspace
    __shared__ BwdSmem<N> sm;

    const int bh = blockIdx.x / Geo::P, part = blockIdx.x - bh * Geo::P;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = p.T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane / Geo::LR, cg = lane % Geo::LR;
    const int il0 = Geo::RW * wave + 4 * rg;  // this lane's rows within the workgroup's band
    const int i0 = Geo::RB * part + il0;      // value rows i0 .. i0+3
    const int j0 = 4 * cg;                    // key columns j0 .. j0+3
    const long HN = (long)p.H * N;
    const long tok0 = (long)b * T * HN + (long)h * N;
    const int nck = (T + kCkpt - 1) / kCkpt;
    const float *ckb = p.s_ckpt + (long)bh * nck * N * N + (long)i0 * N + j0;
    const long sb0 = (long)bh * N * N + (long)i0 * N + j0;
    // staging roles: slot q of this thread is token s_t[q], 4-column slice s_q[q]
    int s_t[Geo::SLOTS], s_q[Geo::SLOTS];
#pragma unroll
    for (int q = 0; q < Geo::SLOTS; ++q) {
        const int s = tid + kBwdThreads * q;
        s_t[q] = s / Geo::LR;
        s_q[q] = s % Geo::LR;
    }

    float G[4][4];  // cotangent of the current state
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (sl.g_in) x = *reinterpret_cast<const float4 *>(sl.g_in + sb0 + e * N);
        G[e][0] = x.x; G[e][1] = x.y; G[e][2] = x.z; G[e][3] = x.w;
    }

    typename L::T xr[Geo::SLOTS], xk[Geo::SLOTS], xv[Geo::SLOTS], xkap[Geo::SLOTS];
    typename L::T xa[Geo::SLOTS], xdy[Geo::SLOTS];
    typename LW::T xw[Geo::SLOTS];
    auto issue = [&](int c) {
#pragma unroll
        for (int q = 0; q < Geo::SLOTS; ++q) {
            const int t = c * kCkpt + s_t[q];
            if (t < T) {
                const long off = tok0 + (long)t * HN + 4 * s_q[q];
                xr[q] = L::load(p.r, off);
                xw[q] = LW::load(p.w, off);
                xk[q] = L::load(p.k, off);
                xv[q] = L::load(p.v, off);
                xkap[q] = L::load(p.kappa, off);
                xa[q] = L::load(p.a, off);
                xdy[q] = L::load(p.dy, off);
            } else {
                xr[q] = xk[q] = xv[q] = xkap[q] = xa[q] = xdy[q] = L::zero();
                xw[q] = LW::zero();
            }
        }
    };
    float4 ckn[4];
    auto issue_ck = [&](int c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ckn[e] = *reinterpret_cast<const float4 *>(ckb + (long)c * N * N + e * N);
    };

    // one token forward: S <- S diag(w) - u b^T + v k^T, u = S kappa (returned)
    auto step = [&](float (&S)[4][4], int t, float (&u)[4]) {
        const float4 kp = lds4(&sm.kap[t][j0]), w4 = lds4(&sm.w[t][j0]);
        const float4 b4 = lds4(&sm.b[t][j0]), k4 = lds4(&sm.k[t][j0]);
        const float4 v4 = lds4(&sm.v[t][il0]);
        const float wq[4] = {w4.x, w4.y, w4.z, w4.w}, bq[4] = {b4.x, b4.y, b4.z, b4.w};
        const float kq[4] = {k4.x, k4.y, k4.z, k4.w}, ve[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = row_sum<N>(S[e][0] * kp.x + S[e][1] * kp.y + S[e][2] * kp.z + S[e][3] * kp.w);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) S[e][q] = S[e][q] * wq[q] - u[e] * bq[q] + ve[e] * kq[q];
    };

    issue(sl.c_end - 1);
    issue_ck(sl.c_end - 1);
    int buf = 0;
    for (int c = sl.c_end - 1; c >= sl.c_begin; --c) {
        const int tb = c * kCkpt;
        float C0[4][4];  // the stored state before token tb
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            C0[e][0] = ckn[e].x; C0[e][1] = ckn[e].y; C0[e][2] = ckn[e].z; C0[e][3] = ckn[e].w;
        }
        __syncthreads();  // the previous interval's last block is written out
        // ---- stage this interval's vectors (fp32; padding: w = 1, rest 0) ----
#pragma unroll
        for (int q = 0; q < Geo::SLOTS; ++q) {
            float4 w4 = LW::widen(xw[q]);
            if (tb + s_t[q] >= T) w4 = make_float4(1.f, 1.f, 1.f, 1.f);
            const float4 r4 = L::widen(xr[q]), k4 = L::widen(xk[q]), v4 = L::widen(xv[q]);
            const float4 kp4 = L::widen(xkap[q]), a4 = L::widen(xa[q]), dy4 = L::widen(xdy[q]);
            const float4 b4 =
                make_float4(a4.x * kp4.x, a4.y * kp4.y, a4.z * kp4.z, a4.w * kp4.w);
            const int st = s_t[q], sc = 4 * s_q[q];
            const int sv = sc - Geo::RB * part;  // value channel within the band
            *reinterpret_cast<float4 *>(&sm.r[st][sc]) = r4;
            *reinterpret_cast<float4 *>(&sm.w[st][sc]) = w4;
            *reinterpret_cast<float4 *>(&sm.k[st][sc]) = k4;
            *reinterpret_cast<float4 *>(&sm.kap[st][sc]) = kp4;
            if constexpr (!kPart) *reinterpret_cast<float4 *>(&sm.a[st][sc]) = a4;
            *reinterpret_cast<float4 *>(&sm.b[st][sc]) = b4;
            if (!kPart || (unsigned)sv < (unsigned)Geo::RB) {
                *reinterpret_cast<float4 *>(&sm.v[st][sv]) = v4;
                *reinterpret_cast<float4 *>(&sm.dy[st][sv]) = dy4;
            }
        }
        __syncthreads();
        if (c > sl.c_begin) {
            issue(c - 1);
            issue_ck(c - 1);
        }

        float S4[4][4], S8[4][4];  // the states before tokens 4 and 8
        for (int blk = kNBlk - 1; blk >= 0; --blk) {
            const int t0 = kBlk * blk;
            // ---- recompute: the states before tokens t0 .. t0+3 ----
            // (the last block walks from the stored state and keeps the states
            // before tokens 4 and 8 for the blocks after it)
            float S[4][4];
            float u[kBlk][4];
            if (blk == kNBlk - 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) S[e][q] = C0[e][q];
                for (int t = 0; t < 4; ++t) step(S, t, u[0]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) S4[e][q] = S[e][q];
                for (int t = 4; t < 8; ++t) step(S, t, u[0]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) S8[e][q] = S[e][q];
                for (int t = 8; t < 12; ++t) step(S, t, u[0]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        S[e][q] = blk == 2 ? S8[e][q] : (blk == 1 ? S4[e][q] : C0[e][q]);
            }
            static_assert(kNBlk == 4, "the walk above keeps the states of blocks 1 and 2");
            float Sp[kBlk][4][4];
#pragma unroll
            for (int tt = 0; tt < kBlk; ++tt) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) Sp[tt][e][q] = S[e][q];
                step(S, t0 + tt, u[tt]);
            }
            // S is now the state after token t0+3

            // ---- tokens t0+3 .. t0, backwards ----
#pragma unroll
            for (int tt = kBlk - 1; tt >= 0; --tt) {
                const int t = t0 + tt;
                const float4 r4t = lds4(&sm.r[t][j0]), w4t = lds4(&sm.w[t][j0]);
                const float4 k4t = lds4(&sm.k[t][j0]), kp4t = lds4(&sm.kap[t][j0]);
                const float4 b4t = lds4(&sm.b[t][j0]);
                const float4 v4t = lds4(&sm.v[t][il0]), dy4t = lds4(&sm.dy[t][il0]);
                const float rq[4] = {r4t.x, r4t.y, r4t.z, r4t.w};
                const float wq[4] = {w4t.x, w4t.y, w4t.z, w4t.w};
                const float kq[4] = {k4t.x, k4t.y, k4t.z, k4t.w};
                const float kpq[4] = {kp4t.x, kp4t.y, kp4t.z, kp4t.w};
                const float bq[4] = {b4t.x, b4t.y, b4t.z, b4t.w};
                const float ve[4] = {v4t.x, v4t.y, v4t.z, v4t.w};
                const float dye[4] = {dy4t.x, dy4t.y, dy4t.z, dy4t.w};
                // S_t (after token t) and S_{t-1} (before it)
                float St[4][4], Sm[4][4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        St[e][q] = (tt == kBlk - 1) ? S[e][q] : Sp[(tt + 1) % kBlk][e][q];
                        Sm[e][q] = Sp[tt][e][q];
                    }

#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) G[e][q] += dye[e] * rq[q];
                float cs[kNCol][4];  // column sums over this lane's 4 rows
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float s_r = 0.f, s_k = 0.f, s_b = 0.f, s_w = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        s_r += St[e][q] * dye[e];
                        s_k += G[e][q] * ve[e];
                        s_b -= G[e][q] * u[tt][e];
                        s_w += G[e][q] * Sm[e][q];
                    }
                    cs[0][q] = s_r; cs[1][q] = s_k; cs[2][q] = s_b; cs[3][q] = s_w;
                }
                float dv[4], du[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dv[e] = row_sum<N>(G[e][0] * kq[0] + G[e][1] * kq[1] + G[e][2] * kq[2] +
                                       G[e][3] * kq[3]);
                    du[e] = -row_sum<N>(G[e][0] * bq[0] + G[e][1] * bq[1] + G[e][2] * bq[2] +
                                        G[e][3] * bq[3]);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    cs[4][q] = Sm[0][q] * du[0] + Sm[1][q] * du[1] + Sm[2][q] * du[2] +
                               Sm[3][q] * du[3];
                // cotangent of the state before token t
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q) G[e][q] = G[e][q] * wq[q] + du[e] * kpq[q];
                // column sums over the wave's rows
                const int ct = kPart ? 0 : tt;  // token slot of the write-out buffer
#pragma unroll
                for (int x = 0; x < kNCol; ++x) {
                    if constexpr (N == 64) {
                        // four row groups, four columns per register: lanes of row
                        // group rg end with column j0 + packed_col(rg)
                        const float s4 = sum_rows4_packed(cs[x][0], cs[x][1], cs[x][2], cs[x][3]);
                        sm.col[buf][wave][ct][x][j0 + packed_col(rg)] = s4;
                    } else {
                        // two row groups (lane bit 5): rg 0 ends with columns j0 and
                        // j0 + 2, rg 1 with j0 + 1 and j0 + 3
                        sm.col[buf][wave][ct][x][j0 + rg] = swap32_add(cs[x][0], cs[x][1]);
                        sm.col[buf][wave][ct][x][j0 + 2 + rg] = swap32_add(cs[x][2], cs[x][3]);
                    }
                }
                if (cg == 0)
                    *reinterpret_cast<float4 *>(&sm.dv[buf][ct][il0]) =
                        make_float4(dv[0], dv[1], dv[2], dv[3]);
                if constexpr (kPart) {
                    // ---- this token's partial column sums (float32) and dv ----
                    __syncthreads();
                    const int tg = tb + t;
                    if (tg < T) {
                        const long plane = (long)p.B * sl.L * HN;  // elements per (sum, part)
                        const long pbase =
                            ((long)b * sl.L + (tg - sl.c_begin * kCkpt)) * HN + (long)h * N;
                        for (int e = tid; e < kNCol * N; e += kBwdThreads) {
                            const int x = e / N, j = e % N;
                            sl.part[(long)(x * Geo::P + part) * plane + pbase + j] =
                                (sm.col[buf][0][0][x][j] + sm.col[buf][1][0][x][j]) +
                                (sm.col[buf][2][0][x][j] + sm.col[buf][3][0][x][j]);
                        }
                        // dv is a row sum: complete for the band's rows
                        if (tid < Geo::RB)
                            IO::store1(static_cast<E *>(p.dv) + tok0 + (long)tg * HN +
                                           Geo::RB * part + tid,
                                       sm.dv[buf][0][tid]);
                    }
                    buf ^= 1;
                }
            }

            // ---- write out the block's gradients: thread = (token, channel) ----
            if constexpr (!kPart) {
                __syncthreads();
                const int tt = tid >> 6, j = tid & 63;
                const int t = tb + t0 + tt;
                if (t < T) {
                    float s[kNCol];
#pragma unroll
                    for (int x = 0; x < kNCol; ++x)
                        s[x] = (sm.col[buf][0][tt][x][j] + sm.col[buf][1][tt][x][j]) +
                               (sm.col[buf][2][tt][x][j] + sm.col[buf][3][tt][x][j]);
                    const float kj = sm.kap[t0 + tt][j], aj = sm.a[t0 + tt][j];
                    const long o = tok0 + (long)t * HN + j;
                    IO::store1(static_cast<E *>(p.dr) + o, s[0]);
                    IO::store1(static_cast<E *>(p.dk) + o, s[1]);
                    IOW::store1(static_cast<EW *>(p.dw) + o, s[3]);
                    IO::store1(static_cast<E *>(p.dkappa) + o, s[4] + aj * s[2]);
                    IO::store1(static_cast<E *>(p.da) + o, kj * s[2]);
                    IO::store1(static_cast<E *>(p.dv) + o, sm.dv[buf][tt][j]);
                }
                buf ^= 1;
            }
        }
    }

    if (sl.g_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<float4 *>(sl.g_out + sb0 + e * N) =
                make_float4(G[e][0], G[e][1], G[e][2], G[e][3]);
    }
}

// N = 128: add the four bands' partial column sums of tokens [t_begin,
// t_begin + len) in a fixed order and form the gradients.  Thread = four
// consecutive channels of one (b, t, h).
template <class IO, bool W32>
__global__ __launch_bounds__(kCombineThreads) void backward_combine_kernel(BackwardArgs p,
                                                                          BwdSlice sl,
                                                                          int t_begin, int len) {
    constexpr int N = 128, P = BwdGeo<N>::P;
    using IOW = std::conditional_t<W32, F32In, IO>;
    using E = typename IO::elem;
    using EW = typename IOW::elem;
    const long HN = (long)p.H * N;
    const long n4 = (long)p.B * len * HN / 4;
    const long e4 = (long)blockIdx.x * kCombineThreads + threadIdx.x;
    if (e4 >= n4) return;
    const long el = 4 * e4;
    const long bt = el / HN, rem = el - bt * HN;  // bt = b * len + tl; rem = h * N + j
    const long b = bt / len, tl = bt - b * len;
    const long o = (b * p.T + t_begin + tl) * HN + rem;
    const long po = (b * sl.L + tl) * HN + rem;
    const long plane = (long)p.B * sl.L * HN;
    float4 s[kNCol];
#pragma unroll
    for (int x = 0; x < kNCol; ++x) {
        s[x] = *reinterpret_cast<const float4 *>(sl.part + (long)(x * P) * plane + po);
#pragma unroll
        for (int q = 1; q < P; ++q) {
            const float4 y = *reinterpret_cast<const float4 *>(sl.part + (long)(x * P + q) * plane + po);
            s[x] = make_float4(s[x].x + y.x, s[x].y + y.y, s[x].z + y.z, s[x].w + y.w);
        }
    }
    const float4 a4 = IO::load4(static_cast<const E *>(p.a) + o);
    const float4 k4 = IO::load4(static_cast<const E *>(p.kappa) + o);
    const float4 db = s[2];
    IO::store4(static_cast<E *>(p.dr) + o, s[0]);
    IO::store4(static_cast<E *>(p.dk) + o, s[1]);
    IOW::store4(static_cast<EW *>(p.dw) + o, s[3]);
    IO::store4(static_cast<E *>(p.dkappa) + o,
               make_float4(s[4].x + a4.x * db.x, s[4].y + a4.y * db.y, s[4].z + a4.z * db.z,
                           s[4].w + a4.w * db.w));
    IO::store4(static_cast<E *>(p.da) + o,
               make_float4(k4.x * db.x, k4.y * db.y, k4.z * db.z, k4.w * db.w));
}

// N = 128: tokens per slice, so that the partial sums of one slice stay within
// kPartCap bytes (at least one interval per slice).
constexpr size_t kPartCap = size_t(256) << 20;

size_t part_bytes_per_token(int B, int H) {
    return (size_t)kNCol * BwdGeo<128>::P * B * H * 128 * sizeof(float);
}

int slice_tokens(int B, int T, int H) {
    size_t L = kPartCap / part_bytes_per_token(B, H) / kCkpt * kCkpt;
    if (L < (size_t)kCkpt) L = kCkpt;
    const size_t Tp = ((size_t)T + kCkpt - 1) / kCkpt * kCkpt;
    return (int)(L < Tp ? L : Tp);
}

template <class IO, bool W32, int N>
hipError_t launch_slices(const BackwardArgs &p, hipStream_t stream) {
    const int nck = (p.T + kCkpt - 1) / kCkpt;
    const long bh = (long)p.B * p.H;
    if constexpr (N == 64) {
        const BwdSlice sl{0, nck, p.ds_T, p.ds0, nullptr, 0};
        hipLaunchKernelGGL((backward_kernel<IO, W32, 64>), dim3((unsigned)bh), dim3(kBwdThreads),
                           0, stream, p, sl);
        return hipGetLastError();
    } else {
        const int L = slice_tokens(p.B, p.T, p.H);
        const int nslice = (p.T + L - 1) / L;
        float *part = p.scan_ws;
        float *carry = part + part_bytes_per_token(p.B, p.H) * L / sizeof(float);
        for (int si = nslice - 1; si >= 0; --si) {
            BwdSlice sl{};
            sl.c_begin = si * (L / kCkpt);
            sl.c_end = min((si + 1) * (L / kCkpt), nck);
            sl.g_in = si == nslice - 1 ? p.ds_T : carry;
            sl.g_out = si == 0 ? p.ds0 : carry;
            sl.part = part;
            sl.L = L;
            hipLaunchKernelGGL((backward_kernel<IO, W32, 128>),
                               dim3((unsigned)(bh * BwdGeo<128>::P)), dim3(kBwdThreads), 0,
                               stream, p, sl);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            const int t_begin = si * L, len = min(L, p.T - t_begin);
            const long n4 = (long)p.B * len * p.H * (128 / 4);
            hipLaunchKernelGGL((backward_combine_kernel<IO, W32>),
                               dim3((unsigned)((n4 + kCombineThreads - 1) / kCombineThreads)),
                               dim3(kCombineThreads), 0, stream, p, sl, t_begin, len);
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
}

template <int N>
hipError_t launch_backward_n(const BackwardArgs &p, hipStream_t stream) {
    if (p.w32) return launch_slices<Bf16In, true, N>(p, stream);
    if (p.bf16) return launch_slices<Bf16In, false, N>(p, stream);
    return launch_slices<F32In, false, N>(p, stream);
}

}  // namespace

size_t backward_scan_workspace_bytes(int B, int T, int H, int N) {
    if (N != 128 || T <= 0) return 0;
    const int L = slice_tokens(B, T, H);
    size_t n = part_bytes_per_token(B, H);
    if (n > SIZE_MAX / (size_t)L) return 0;
    n *= (size_t)L;
    if ((T + L - 1) / L > 1) {  // the carried cotangent between slices
        const size_t carry = (size_t)B * H * 128 * 128 * sizeof(float);
        if (n > SIZE_MAX - carry) return 0;
        n += carry;
    }
    return n;
}

hipError_t launch_backward(const BackwardArgs &p, hipStream_t stream) {
    return p.N == 128 ? launch_backward_n<128>(p, stream) : launch_backward_n<64>(p, stream);
}

}  // namespace wkv7
