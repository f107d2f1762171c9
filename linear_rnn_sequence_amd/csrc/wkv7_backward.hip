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
// Work split.  One workgroup (4 waves) per (batch, head).  Value rows are
// independent in both directions (row i of S and of G only meets v_i, u_i,
// dy_i, du_i), so wave w owns rows 16w .. 16w+15, and lane (rg, cg) holds rows
// 16w + 4rg .. +3 and key columns 4cg .. 4cg+3 of S, of the recomputed states
// and of G.  Row sums (u, dv, du) are 16-lane DPP reductions; the column sums
// (dr, dk, db, dw and the S^T du part of dkappa) are outputs only, so they are
// reduced over the wave's four row groups with permlane swaps and left per
// wave in LDS, and the four waves' parts are added when a block of tokens is
// written out.
//
// Per 16-token interval, in reverse: the interval's inputs and dy are staged
// in LDS as fp32 (the previous interval's loads are in flight meanwhile); then
// for each 4-token block, last first, the states before its tokens are
// recomputed from the interval's stored state, kept in registers, and the four
// tokens are walked backwards.  Padding tokens past T carry w = 1 and zeros
// elsewhere, which leaves S and G unchanged.
#include "wkv7_device.h"
#include "wkv7_internal.h"

namespace wkv7 {
namespace {

constexpr int kBwdThreads = 256;
constexpr int kBlk = 4;                // tokens per recompute block
constexpr int kNBlk = kCkpt / kBlk;    // blocks per interval
constexpr int kNCol = 5;               // column sums: dr, dk, db, dw, S^T du

struct __align__(16) BwdSmem {
    float r[kCkpt][kN], w[kCkpt][kN], k[kCkpt][kN], v[kCkpt][kN];
    float kap[kCkpt][kN], a[kCkpt][kN], b[kCkpt][kN], dy[kCkpt][kN];
    float col[2][4][kBlk][kNCol][kN];  // [buffer][wave][token][sum][column]
    float dv[2][kBlk][kN];             // [buffer][token][row]
};

__device__ __forceinline__ float4 lds4(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
}

template <class IO>
__global__ __launch_bounds__(kBwdThreads) void backward_kernel(BackwardArgs p) {
    using L = RawLoad<IO>;
    using E = typename IO::elem;
    __shared__ BwdSmem sm;

    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H;
    const int T = p.T;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, cg = lane & 15;
    const int i0 = 16 * wave + 4 * rg;  // value rows i0 .. i0+3
    const int j0 = 4 * cg;              // key columns j0 .. j0+3
    const long HN = (long)p.H * kN;
    const long tok0 = (long)b * T * HN + (long)h * kN;
    const int s_t = tid >> 4, s_q = tid & 15;  // staging role: token, 4-column slice
    const int nck = (T + kCkpt - 1) / kCkpt;
    const float *ckb = p.s_ckpt + (long)bh * nck * kN * kN + (long)i0 * kN + j0;
    const long sb0 = (long)bh * kN * kN + (long)i0 * kN + j0;

    float G[4][4];  // cotangent of the current state
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.ds_T) x = *reinterpret_cast<const float4 *>(p.ds_T + sb0 + e * kN);
        G[e][0] = x.x; G[e][1] = x.y; G[e][2] = x.z; G[e][3] = x.w;
    }

    typename L::T xr, xw, xk, xv, xkap, xa, xdy;
    auto issue = [&](int c) {
        const int t = c * kCkpt + s_t;
        if (t < T) {
            const long off = tok0 + (long)t * HN + 4 * s_q;
            xr = L::load(p.r, off);
            xw = L::load(p.w, off);
            xk = L::load(p.k, off);
            xv = L::load(p.v, off);
            xkap = L::load(p.kappa, off);
            xa = L::load(p.a, off);
            xdy = L::load(p.dy, off);
        } else {
            xr = xw = xk = xv = xkap = xa = xdy = L::zero();
        }
    };
    float4 ckn[4];
    auto issue_ck = [&](int c) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ckn[e] = *reinterpret_cast<const float4 *>(ckb + (long)c * kN * kN + e * kN);
    };

    // one token forward: S <- S diag(w) - u b^T + v k^T, u = S kappa (returned)
    auto step = [&](float (&S)[4][4], int t, float (&u)[4]) {
        const float4 kp = lds4(&sm.kap[t][j0]), w4 = lds4(&sm.w[t][j0]);
        const float4 b4 = lds4(&sm.b[t][j0]), k4 = lds4(&sm.k[t][j0]);
        const float4 v4 = lds4(&sm.v[t][i0]);
        const float wq[4] = {w4.x, w4.y, w4.z, w4.w}, bq[4] = {b4.x, b4.y, b4.z, b4.w};
        const float kq[4] = {k4.x, k4.y, k4.z, k4.w}, ve[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            u[e] = sum_lanes16(S[e][0] * kp.x + S[e][1] * kp.y + S[e][2] * kp.z + S[e][3] * kp.w);
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int q = 0; q < 4; ++q) S[e][q] = S[e][q] * wq[q] - u[e] * bq[q] + ve[e] * kq[q];
    };

    issue(nck - 1);
    issue_ck(nck - 1);
    int buf = 0;
    for (int c = nck - 1; c >= 0; --c) {
        const int tb = c * kCkpt;
        // ---- stage this interval's vectors (fp32; padding: w = 1, rest 0) ----
        float4 w4 = L::widen(xw);
        if (tb + s_t >= T) w4 = make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 r4 = L::widen(xr), k4 = L::widen(xk), v4 = L::widen(xv);
        const float4 kp4 = L::widen(xkap), a4 = L::widen(xa), dy4 = L::widen(xdy);
        const float4 b4 = make_float4(a4.x * kp4.x, a4.y * kp4.y, a4.z * kp4.z, a4.w * kp4.w);
        float C0[4][4];  // the stored state before token tb
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            C0[e][0] = ckn[e].x; C0[e][1] = ckn[e].y; C0[e][2] = ckn[e].z; C0[e][3] = ckn[e].w;
        }
        __syncthreads();  // the previous interval's last block is written out
        *reinterpret_cast<float4 *>(&sm.r[s_t][4 * s_q]) = r4;
        *reinterpret_cast<float4 *>(&sm.w[s_t][4 * s_q]) = w4;
        *reinterpret_cast<float4 *>(&sm.k[s_t][4 * s_q]) = k4;
        *reinterpret_cast<float4 *>(&sm.v[s_t][4 * s_q]) = v4;
        *reinterpret_cast<float4 *>(&sm.kap[s_t][4 * s_q]) = kp4;
        *reinterpret_cast<float4 *>(&sm.a[s_t][4 * s_q]) = a4;
        *reinterpret_cast<float4 *>(&sm.b[s_t][4 * s_q]) = b4;
        *reinterpret_cast<float4 *>(&sm.dy[s_t][4 * s_q]) = dy4;
        __syncthreads();
        if (c > 0) {
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
                const float4 v4t = lds4(&sm.v[t][i0]), dy4t = lds4(&sm.dy[t][i0]);
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
                    dv[e] = sum_lanes16(G[e][0] * kq[0] + G[e][1] * kq[1] + G[e][2] * kq[2] +
                                        G[e][3] * kq[3]);
                    du[e] = -sum_lanes16(G[e][0] * bq[0] + G[e][1] * bq[1] + G[e][2] * bq[2] +
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
                // column sums over the wave's 16 rows, four columns per register:
                // lanes of row group rg end with column j0 + kPackedCol[rg]
#pragma unroll
                for (int x = 0; x < kNCol; ++x) {
                    const float s4 = sum_rows4_packed(cs[x][0], cs[x][1], cs[x][2], cs[x][3]);
                    sm.col[buf][wave][tt][x][j0 + packed_col(rg)] = s4;
                }
                if (cg == 0)
                    *reinterpret_cast<float4 *>(&sm.dv[buf][tt][i0]) =
                        make_float4(dv[0], dv[1], dv[2], dv[3]);
            }
            __syncthreads();

            // ---- write out the block's gradients: thread = (token, channel) ----
            {
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
                    IO::store1(static_cast<E *>(p.dw) + o, s[3]);
                    IO::store1(static_cast<E *>(p.dkappa) + o, s[4] + aj * s[2]);
                    IO::store1(static_cast<E *>(p.da) + o, kj * s[2]);
                    IO::store1(static_cast<E *>(p.dv) + o, sm.dv[buf][tt][j]);
                }
            }
            buf ^= 1;
        }
    }

    if (p.ds0) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            *reinterpret_cast<float4 *>(p.ds0 + sb0 + e * kN) =
                make_float4(G[e][0], G[e][1], G[e][2], G[e][3]);
    }
}

}  // namespace

hipError_t launch_backward(const BackwardArgs &p, hipStream_t stream) {
    const dim3 grid((unsigned)((long)p.B * p.H)), block(kBwdThreads);
    if (p.bf16)
        hipLaunchKernelGGL(backward_kernel<Bf16In>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(backward_kernel<F32In>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace wkv7
