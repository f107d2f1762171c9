// WKV7 backward in the chunked form on bf16 MFMA (fp32 accumulation).
//
// The recurrence (RWKV-7 "Goose" author response, numpy time_mixing listing;
// ARWKV verdict, key_machinery field) is, per head, with S[i = value][j = key]
//   S_t = S_{t-1} A_t + v_t k_t^T,   A_t = diag(w_t) - kappa_t (a_t * kappa_t)^T,
//   y_t = S_t r_t,
// and the gradients are those of L = sum_t <y_t, dy_t> + <S_T, dS_T>.  Over a
// chunk of 16 tokens with entry state S0 (the stored checkpoint) the forward is
// (derivation not on the pages; tests/test_chunked_backward_algebra.py checks
// these formulas in fp64 against autograd of the per-token loop):
//   g_t = prod_{s<=t} w_s, gp_t = g_{t-1}; Kp = kappa*gp, Rp = r*g, Km = k/g,
//   Bm = (a*kappa)/g; Mkk = stril(Kp Km^T), N = stril(Kp Bm^T),
//   Mkr = tril(Rp Km^T), Mbr = tril(Rp Bm^T); X = (I + N)^-1 (by block
//   substitution, tri_inverse in wkv7_mfma.h);
//   U = X (Kp S0^T + Mkk V) (the chunk's S_{t-1} kappa_t), Y = Rp S0^T + Mkr V - Mbr U,
//   S_C = (S0 + V^T Km - U^T Bm) diag(g_C).
// Its reverse-mode derivative, with dSh = dS_C diag(g_C) and dS_C the cotangent
// of the chunk's exit state:
//   dU = -Bm dSh^T - Mbr^T dY,  dZ = X^T dU,
//   dS0 = dSh + dY^T Rp + dZ^T Kp                      (the reverse chain)
//   dV = Km dSh^T + Mkr^T dY + Mkk^T dZ
//   dMkr = tril(dY V^T), dMbr = -tril(dY U^T), dMkk = stril(dZ V^T), dMbk = -stril(dZ U^T)
//   dKm = V dSh + dMkr^T Rp + dMkk^T Kp,  dBm = -U dSh + dMbr^T Rp + dMbk^T Kp
//   dRp = dY S0 + dMkr Km + dMbr Bm,      dKp = dZ S0 + dMkk Km + dMbk Bm
// and back to the inputs: dr = dRp g, dk = dKm / g, db = dBm / g, da = db kappa,
// dkappa = dKp gp + db a.  The decays enter only through g: with
//   dlg_t = dRp_t Rp_t - dKm_t Km_t - dBm_t Bm_t + dKp_{t+1} Kp_{t+1}
// (elementwise) plus, at the chunk's last slot, the exit-state term
//   sum_i dS_C S_C = sum_i dSh S0 + sum_s Km_s (V dSh)_s + sum_s Bm_s (-U dSh)_s,
// dw_s = (sum_{t >= s} dlg_t) / w_s.  The same-token parts of dlg_t (from the
// diagonals of dMkr, dMbr and the first sub-diagonals of dMkk, dMbk) cancel
// exactly and are left out (phase 3 of the gradient kernel).
//
// Two kernels:
//  - bwd_chain_kernel: one workgroup per (b, h) walks the chunks backwards and
//    carries dS^T as fp32 MFMA accumulator tiles (wave q owns values 16q..16q+15,
//    like the forward chunked kernel's state); it stores the dSh of the last
//    chunk of every group of 8 in bf16 (the MFMA operand both kernels use) to
//    the workspace and writes ds0;
//  - bwd_grad_kernel: each workgroup takes one such group (8 consecutive chunks
//    of one head) and walks it last to first: from a chunk's stored entry
//    state and dSh it recomputes the chunk's operands and forms every gradient,
//    and the chunk's dS0 (the products the chain kernel forms) gives the
//    earlier chunk's dSh, so the state cotangent crosses the group in fp32
//    registers; it loads the next chunk's inputs while it works on the current
//    one.
//    Its four waves each form a share of the chunk's C x C matrices (X, M_kk,
//    M_kr, M_br, then the cotangent matrices dM) and pass them to the others
//    through LDS as bf16 MFMA operands.
// A ragged last chunk is padded with neutral tokens (w = 1, all else 0), which
// leave every product and the decay totals unchanged.
//
// MFMA layouts (v_mfma_f32_16x16x16_bf16, lane l: lo = l & 15, g = l >> 4):
//   A operand of P (16 x 16):   lane holds P[lo][4g + e]
//   B operand of Q (16 x 16):   lane holds Q[4g + e][lo]
//   result D (16 x 16):         lane holds D[4g + e][lo]
// so D(M) is the B operand of M and the A operand of M^T.  Every operand read
// from LDS below is `frag(M, row0, col0)`, four consecutive bf16 of row
// row0 + lo at columns col0 + 4g: the A operand of a matrix stored with the
// contraction index along its rows, or the B operand of one whose transpose is
// stored that way.
#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {
namespace {

constexpr int kC = 16;        // tokens per chunk (the checkpoint interval)
constexpr int kThreads = 256;  // four waves
constexpr int kSK = 68;       // row stride (bf16) of 16 x 64 and 64 x 64 tiles
constexpr int kST = 20;       // row stride (bf16) of 64 x 16 (transposed) tiles
constexpr int kGradChunks = 8;  // consecutive chunks of one head per gradient workgroup

static_assert(kC == kCkpt, "chunks are the checkpoint intervals");

// every product of this file is a 16x16x16 MFMA: accumulators are Acc16
__device__ __forceinline__ Acc16 mma(bf16x4 a, bf16x4 b, Acc16 c) { return mfma16(a, b, c); }
// two floats -> packed bf16 pair, round to nearest even (the hardware conversion)
__device__ __forceinline__ unsigned cvt2(float lo, float hi) { return cvt_pk(lo, hi); }
__device__ __forceinline__ bf16x4 bf4(f32x4 x) { return to_bf16(x); }
__device__ __forceinline__ bf16x4 bf4(Acc16 x) { return to_bf16(x.v); }
// one float -> bf16 bits, round to nearest even (the same hardware conversion)
__device__ __forceinline__ short bf1(float x) { return (short)(cvt2(x, 0.f) & 0xffffu); }
__device__ __forceinline__ uint16_t bf1u(float x) { return (uint16_t)(cvt2(x, 0.f) & 0xffffu); }
__device__ __forceinline__ float fbf(short s) { return __uint_as_float(((uint32_t)(uint16_t)s) << 16); }
__device__ __forceinline__ Acc16 z4() { return Acc16::zero(); }
__device__ __forceinline__ Acc16 neg(Acc16 x) { return Acc16{-x.v}; }

template <int S>
__device__ __forceinline__ bf16x4 frag(const short (*m)[S], int row0, int col0, int lane) {
    return *reinterpret_cast<const bf16x4 *>(&m[row0 + (lane & 15)][col0 + 4 * (lane >> 4)]);
}

// B operand of a 16-row tile stored row-major (rows = the contraction index):
// rows g4 .. g4+3 of column col0 + lo, four 2-byte reads
template <int S>
__device__ __forceinline__ bf16x4 colfrag(const short (*m)[S], int col0, int lane) {
    const int c = col0 + (lane & 15), r = 4 * (lane >> 4);
    return bf16x4{m[r][c], m[r + 1][c], m[r + 2][c], m[r + 3][c]};
}

// Keep the entries of a result tile D[4g+e][lo] that satisfy a triangle:
// kLower: col <= row (kStrict: col < row); else row <= col (kStrict: row < col).
template <bool kLower, bool kStrict>
__device__ __forceinline__ Acc16 mask(Acc16 d, int lane) {
    const int lo = lane & 15, row = 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = row + e;
        const bool keep = kLower ? (kStrict ? lo < r : lo <= r) : (kStrict ? r < lo : r <= lo);
        d.v[e] = keep ? d[e] : 0.f;
    }
    return d;
}


// mask<kLower, strict>, the strictness a run-time (wave-uniform) value
template <bool kLower>
__device__ __forceinline__ Acc16 mask_rt(Acc16 d, int lane, bool strict) {
    const int lo = lane & 15, row = 4 * (lane >> 4), ofs = strict ? 0 : 1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = row + e;
        const bool keep = kLower ? (lo < r + ofs) : (r < lo + ofs);
        d.v[e] = keep ? d[e] : 0.f;
    }
    return d;
}

// bf16 operand with every element negated (exact: a sign flip)
__device__ __forceinline__ bf16x4 negb(bf16x4 x) { return x ^ (short)0x8000; }

// Element offset of token t of (b, h) in a [B,T,H,64] tensor.
__device__ __forceinline__ long tok_off(const BackwardArgs &p, long b, int h, long t) {
    return ((b * p.T + t) * p.H + h) * kN;
}

// The workspace holds, per (b, h) and group of 8 chunks, the dSh of the group's
// last chunk (64 x 64 bf16, 8 KiB) in the order the
// lanes hold it, not row by row: the four bf16 that lane l of wave q holds of
// key block jb (dSh[16q + (l & 15)][16jb + 4(l >> 4) + e], e < 4) are at
// element 4 (64 (4q + jb) + l), so each store and load instruction moves 512
// contiguous bytes (row by row, it touched sixteen 32-byte pieces).
__device__ __forceinline__ int dsh_tile_offset(int q, int jb, int l) {
    return 4 * (64 * (4 * q + jb) + l);
}

// ---------------------------------------------------------------- reverse chain
// One workgroup of nine waves per (b, h) walks the chunks from the last to the
// first as a three-stage pipeline with one barrier per interval (as the
// forward chunked kernel does).  At interval q, with i = q - 2 the chain index
// of the chunk whose cotangent step runs (chunk nch - 1 - i):
//   waves 4..7 ("prep"): wave 4+b forms the operands of tokens 4b .. 4b+3 of
//     chain index q (one token per DPP row, four keys per lane, so each load
//     reads whole token rows), writes them to buffer q % 3, and issues the
//     loads of index q + 3 into its three-deep register ring; at the end it
//     multiplies the decays of index q + 1 over its four tokens and leaves the
//     total in LDS for the later waves (read after the barrier);
//   wave 8 ("matrix"): forms X = (I + N)^-1 and Mbr of index q - 1 from buffer
//     (q - 1) % 3 into the matrix tiles of parity (q - 1) & 1;
//   waves 0..3 ("chain"): wave c owns values 16c .. 16c+15 of dS^T as fp32 MFMA
//     accumulator tiles and runs the cotangent step of index q - 2 from buffer
//     (q - 2) % 3 and the matrix tiles of parity q & 1: it forms the chunk's
//     dSh (bf16 at a group's last chunk, the operand the gradient kernel reads,
//     stored) and dS0.
// Every load is issued on every path (chunk indices clamped), so the ring's
// wait counts stay exact.
constexpr int kChainThreads = 576;  // 4 chain waves + 4 prep waves + 1 matrix wave
// s_waitcnt immediate: vmcnt(0) only (expcnt and lgkmcnt unlimited)
constexpr int kWaitAllLoads = (0x7 << 4) | (0xF << 8);

struct __align__(16) ChainOps {
    short kp[kC][kSK], rp[kC][kSK], bm[kC][kSK];  // tokens x keys
    short kpt[kN][kST], rpt[kN][kST];             // keys x tokens
    short dyt[kN][kST];                           // values x tokens
    float gc[kN];                                 // decay total of the chunk
};
struct __align__(16) ChainMatTiles {
    short xa[kC][kST];    // A operand of X^T: [lo][4g + e] = X[4g + e][lo]
    short mbra[kC][kST];  // A operand of Mbr^T: [lo][4g + e] = Mbr[4g + e][lo]
};
struct __align__(16) ChainLds {
    ChainOps o[3];
    ChainMatTiles m[2];
    float carry[2][4][kN];  // per index parity: decay product of each prep wave's 4 tokens
};

// raw inputs of one chain index held by a prep lane: keys (values) 4lo .. 4lo+3
// of its token, as four bf16 (the decay as four float32 with W32)
template <bool W32> struct ChainRawW { using type = uint2; };
template <> struct ChainRawW<true> { using type = float4; };
template <bool W32>
struct ChainRaw {
    typename ChainRawW<W32>::type w;
    uint2 k, a, r, d;  // kappa, a, r, dy
};

template <bool W32>
__global__ __launch_bounds__(kChainThreads) void bwd_chain_kernel(BackwardArgs p) {
    __shared__ ChainLds L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lo = lane & 15, g4 = 4 * (lane >> 4);
    const long bh = blockIdx.x;
    const long b = bh / p.H;
    const int h = (int)(bh % p.H);
    const int nch = (p.T + kC - 1) / kC;
    const int ngrp = (nch + kGradChunks - 1) / kGradChunks;  // gradient groups (workspace slots)
    const int S = (nch + 7) / 6 * 6;  // intervals: nch + 2, rounded up to whole loop trips

    if (wave < 4) {
        // ---------------- chain waves ----------------
        // dS^T tiles: St[jb] holds dS^T[16jb + g4 + e][16 wave + lo] = dS[16 wave + lo][16jb + g4 + e]
        Acc16 St[4];
        const long srow = (long)(16 * wave + lo) * kN;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            if (p.ds_T) {
                const float4 x =
                    *reinterpret_cast<const float4 *>(p.ds_T + bh * kN * kN + srow + 16 * jb + g4);
                St[jb] = Acc16{f32x4{x.x, x.y, x.z, x.w}};
            } else {
                St[jb] = z4();
            }
        }
        // the state cotangent is in registers before the loop: a load still in
        // flight at its head would make the compiler wait for every vector memory
        // operation there, the previous chunk's dSh stores included (on this
        // target stores count in the same counter as loads)
        __builtin_amdgcn_s_waitcnt(kWaitAllLoads);
        __syncthreads();  // the decay totals of index 0
        for (int q = 0; q < S; ++q) {
            const int i = q - 2;
            if (i >= 0 && i < nch) {
                const int c = nch - 1 - i;
                const ChainOps &o = L.o[i % 3];
                const ChainMatTiles &mt = L.m[i & 1];
                // dSh = dS_C diag(g_C), then dS0 of the chunk.  The last chunk of
                // each gradient group stores its dSh (bf16, the MFMA operand) in
                // the group's workspace slot; the gradient kernel carries the
                // cotangent through the group's other chunks itself.
                bf16x4 Sb[4];
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    const float4 gc = *reinterpret_cast<const float4 *>(&o.gc[16 * jb + g4]);
                    St[jb].v[0] *= gc.x;
                    St[jb].v[1] *= gc.y;
                    St[jb].v[2] *= gc.z;
                    St[jb].v[3] *= gc.w;
                    Sb[jb] = bf4(St[jb]);  // B operand of dSh^T (keys x values)
                }
                if (c % kGradChunks == kGradChunks - 1 || c == nch - 1) {
                    uint16_t *ck = p.ds_ws + (bh * ngrp + c / kGradChunks) * (long)(kN * kN);
#pragma unroll
                    for (int jb = 0; jb < 4; ++jb)
                        *reinterpret_cast<bf16x4 *>(ck + dsh_tile_offset(wave, jb, lane)) = Sb[jb];
                }
                const bf16x4 dyb = frag(o.dyt, 16 * wave, 0, lane);  // B operand of dY (tokens x values)
                Acc16 rhs = mma(frag(mt.mbra, 0, 0, lane), dyb, z4());  // Mbr^T dY
#pragma unroll
                for (int jb = 0; jb < 4; ++jb)
                    rhs = mma(frag(o.bm, 0, 16 * jb, lane), Sb[jb], rhs);  // + Bm dSh^T
                const Acc16 up = mma(frag(mt.xa, 0, 0, lane), bf4(rhs), z4());  // X^T rhs = -dZ
                const bf16x4 dzb = bf4(neg(up));
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    St[jb] = mma(frag(o.rpt, 16 * jb, 0, lane), dyb, St[jb]);  // + Rp^T dY
                    St[jb] = mma(frag(o.kpt, 16 * jb, 0, lane), dzb, St[jb]);  // + Kp^T dZ
                }
            }
            __syncthreads();
        }
        if (p.ds0) {
#pragma unroll
            for (int jb = 0; jb < 4; ++jb)
                *reinterpret_cast<float4 *>(p.ds0 + bh * kN * kN + srow + 16 * jb + g4) =
                    make_float4(St[jb][0], St[jb][1], St[jb][2], St[jb][3]);
        }
        return;
    }

    if (wave == 8) {
        // ---------------- matrix wave: X = (I + N)^-1 and Mbr of index q - 1 ----------------
        // (the interval's critical path: the prep waves' operand formation runs
        // beside it on the other SIMDs)
        __builtin_amdgcn_s_setprio(2);
        __syncthreads();  // the decay totals of index 0
        for (int q = 0; q < S; ++q) {
            const int i = q - 1;
            if (i >= 0 && i < nch) {
                const ChainOps &o = L.o[i % 3];
                ChainMatTiles &mt = L.m[i & 1];
                Acc16 dn = z4(), dnt = z4(), dmbr = z4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const bf16x4 kpa = frag(o.kp, 0, 16 * kb, lane), bma = frag(o.bm, 0, 16 * kb, lane);
                    dn = mma(kpa, bma, dn);    // D(N), N = Kp Bm^T
                    dnt = mma(bma, kpa, dnt);  // D(N^T)
                    dmbr = mma(frag(o.rp, 0, 16 * kb, lane), bma, dmbr);  // D(Mbr), Mbr = Rp Bm^T
                }
                *reinterpret_cast<bf16x4 *>(&mt.mbra[lo][g4]) = bf4(mask<true, false>(dmbr, lane));
                f32x4 dx, dxt;  // D(X) = A operand of X^T (D(X^T) unused here)
                tri_inverse(mask<true, true>(dn, lane).v, mask<false, true>(dnt, lane).v, lane, dx,
                            dxt);
                *reinterpret_cast<bf16x4 *>(&mt.xa[lo][g4]) = bf4(dx);
            }
            __syncthreads();
        }
        return;
    }

    // ---------------- prep waves ----------------
    // Token-major lanes: prep wave pb holds tokens 4pb .. 4pb+3 of a chunk, one
    // per DPP row g, and lane lo of the row keys (values) 4lo .. 4lo+3, so each
    // load instruction reads four whole 128-byte token rows.
    const int pb = wave - 4, t_in = 4 * pb + (lane >> 4), k0 = 4 * lo;
    const long TSH = (long)p.H * kN;  // elements from one token to the next
    // Issues the same loads on every path: the index is clamped to the last one
    // and the token to T - 1, which keeps every address inside the tensors;
    // prep() replaces the values of tokens past T.
    auto load = [&](int i, ChainRaw<W32> &x) {
        const int c = nch - 1 - min(i, nch - 1);
        // the chunk's first token, key 0 (uniform), and the lane's offset from it
        const long base = ((b * p.T + (long)c * kC) * p.H + h) * kN;
        const long o = (long)min(t_in, p.T - 1 - c * kC) * TSH + k0;
        x.r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.r) + base + o);
        if constexpr (W32)
            x.w = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.w) + base + o);
        else
            x.w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.w) + base + o);
        x.k = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.kappa) + base + o);
        x.a = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.a) + base + o);
        x.d = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.dy) + base + o);
    };
    // the lane's four decays of index i (1 past T)
    auto decays = [&](int i, const ChainRaw<W32> &x, float (&w)[4]) {
        const bool ok = (nch - 1 - min(i, nch - 1)) * kC + t_in < p.T;
        if constexpr (W32) {
            w[0] = x.w.x; w[1] = x.w.y; w[2] = x.w.z; w[3] = x.w.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = ok ? w[e] : 1.f;
        } else {
            const unsigned w01 = ok ? x.w.x : 0x3F803F80u, w23 = ok ? x.w.y : 0x3F803F80u;
            w[0] = bf16_lo(w01); w[1] = bf16_hi(w01); w[2] = bf16_lo(w23); w[3] = bf16_hi(w23);
        }
    };
    // Products of w over the wave's four tokens (the DPP rows) for the lane's
    // keys: lp inclusive, lx exclusive.  Row pairs by v_permlane16_swap (its two
    // results hold rows 2k and 2k+1 of the pair k), then the pair (0, 1) total
    // into rows 2, 3 by v_permlane32_swap (its first result holds, in the upper
    // rows, the lower rows of the second operand).
    const bool odd = (lane >> 4) & 1, upper = lane >= 32;
    auto scan = [&](const float (&w)[4], float (&lp)[4], float (&lx)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[e]),
                                                              __float_as_uint(w[e]), false, false);
            const float h0 = __uint_as_float(h16[0]), h1 = __uint_as_float(h16[1]);
            const float pair = h0 * h1;
            const float in1 = odd ? pair : h0;
            const float ex1 = odd ? h0 : 1.f;
            const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair),
                                                              __float_as_uint(pair), false, false);
            const float below = upper ? __uint_as_float(h32[0]) : 1.f;
            lp[e] = in1 * below;
            lx[e] = ex1 * below;
        }
    };
    // the decay products of index i over the wave's four tokens (kept for its
    // operands one interval later) and the wave's total (row 3's inclusive
    // product) into LDS
    struct Scan {
        float lp[4], lx[4];
    };
    auto total = [&](int i, const ChainRaw<W32> &x, Scan &sc) {
        float w[4];
        decays(i, x, w);
        scan(w, sc.lp, sc.lx);
        if (lane >= 48)
            *reinterpret_cast<float4 *>(&L.carry[i & 1][pb][k0]) =
                make_float4(sc.lp[0], sc.lp[1], sc.lp[2], sc.lp[3]);
    };
    // operands of index i into buffer i % 3
    auto prep = [&](int i, const ChainRaw<W32> &x, const Scan &sc) {
        const int c = nch - 1 - min(i, nch - 1);
        const bool ok = c * kC + t_in < p.T;
        ChainOps &o = L.o[i % 3];
        const float *lp = sc.lp, *lx = sc.lx;
        const unsigned k01 = ok ? x.k.x : 0u, k23 = ok ? x.k.y : 0u;
        const unsigned a01 = ok ? x.a.x : 0u, a23 = ok ? x.a.y : 0u;
        const unsigned r01 = ok ? x.r.x : 0u, r23 = ok ? x.r.y : 0u;
        const float kv[4] = {bf16_lo(k01), bf16_hi(k01), bf16_lo(k23), bf16_hi(k23)};
        const float av[4] = {bf16_lo(a01), bf16_hi(a01), bf16_lo(a23), bf16_hi(a23)};
        const float rv[4] = {bf16_lo(r01), bf16_hi(r01), bf16_lo(r23), bf16_hi(r23)};
        const uint2 dyb = ok ? x.d : make_uint2(0u, 0u);
        // decay of the chunk's tokens before this wave's four: the earlier waves'
        // totals (pb is the same over the wave, so the tests are scalar branches)
        const float4(*cw)[kN / 4] = reinterpret_cast<const float4(*)[kN / 4]>(L.carry[i & 1]);
        float4 pre = make_float4(1.f, 1.f, 1.f, 1.f);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            if (q < pb) {
                const float4 y = cw[q][lo];
                pre.x *= y.x; pre.y *= y.y; pre.z *= y.z; pre.w *= y.w;
            }
        }
        if (pb == 0 && lane < 16) {  // the chunk's total, from all four waves
            float4 tot = cw[0][lo];
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                const float4 y = cw[q][lo];
                tot.x *= y.x; tot.y *= y.y; tot.z *= y.z; tot.w *= y.w;
            }
            *reinterpret_cast<float4 *>(&o.gc[k0]) = tot;
        }
        f32x4 Kp, Rp, Bm;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float pr = (&pre.x)[e];
            const float gam = pr * lp[e], gprev = pr * lx[e];
            Kp[e] = kv[e] * gprev;
            Rp[e] = rv[e] * gam;
            Bm[e] = av[e] * kv[e] * __builtin_amdgcn_rcpf(gam);
        }
        const bf16x4 kpb = bf4(Kp), rpb = bf4(Rp);
        *reinterpret_cast<bf16x4 *>(&o.kp[t_in][k0]) = kpb;
        *reinterpret_cast<bf16x4 *>(&o.rp[t_in][k0]) = rpb;
        *reinterpret_cast<bf16x4 *>(&o.bm[t_in][k0]) = bf4(Bm);
        // the transposed tiles: keys (values) k0 .. k0+3 at this token's column
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            o.kpt[k0 + e][t_in] = kpb[e];
            o.rpt[k0 + e][t_in] = rpb[e];
        }
        o.dyt[k0 + 0][t_in] = (short)(dyb.x & 0xffffu);
        o.dyt[k0 + 1][t_in] = (short)(dyb.x >> 16);
        o.dyt[k0 + 2][t_in] = (short)(dyb.y & 0xffffu);
        o.dyt[k0 + 3][t_in] = (short)(dyb.y >> 16);
    };
    // s_waitcnt immediate letting the loads of two indices (five per lane each)
    // stay in flight: vmcnt = 10 (gfx9 encoding: vmcnt[3:0] + vmcnt[5:4] at bits
    // 15:14), expcnt and lgkmcnt unlimited
    constexpr int kLoads = 10;
    constexpr int kWaitTwoIndices = (kLoads & 0xF) | (0x7 << 4) | (0xF << 8) | (((kLoads >> 4) & 0x3) << 14);

    // the ring: index q in xs[q % 3], loaded three intervals ahead (one interval
    // of loads did not cover the memory latency)
    ChainRaw<W32> xs[3];
    Scan sc[2];  // the decay products of the index being prepared and of the next
    load(0, xs[0]);
    load(1, xs[1]);
    load(2, xs[2]);
    __builtin_amdgcn_s_waitcnt(kWaitTwoIndices);  // index 0 in registers
    total(0, xs[0], sc[0]);
    __syncthreads();  // the decay totals of index 0
    // interval q: operands of q, loads of q + 3, totals of q + 1
    auto interval = [&](int q, ChainRaw<W32> &cur, ChainRaw<W32> &nxt, const Scan &scur,
                        Scan &snxt) {
        prep(q, cur, scur);
        load(q + 3, cur);
        __builtin_amdgcn_s_waitcnt(kWaitTwoIndices);  // index q + 1 in registers
        total(q + 1, nxt, snxt);
        __syncthreads();
    };
    for (int q = 0; q < S; q += 6) {  // (S is a multiple of 6)
        interval(q, xs[0], xs[1], sc[0], sc[1]);
        interval(q + 1, xs[1], xs[2], sc[1], sc[0]);
        interval(q + 2, xs[2], xs[0], sc[0], sc[1]);
        interval(q + 3, xs[0], xs[1], sc[1], sc[0]);
        interval(q + 4, xs[1], xs[2], sc[0], sc[1]);
        interval(q + 5, xs[2], xs[0], sc[1], sc[0]);
    }
}

// ------------------------------------------------------- per-chunk gradients
struct GradLds {
    short kp[kC][kSK], rp[kC][kSK], km[kC][kSK], bm[kC][kSK];   // tokens x keys
    short vv[kC][kSK], dyy[kC][kSK], uu[kC][kSK], dzz[kC][kSK];  // tokens x values
    union {
        struct {
            short s0t[kN][kSK], dsht[kN][kSK];  // keys x values (phases 2-3)
        } m;
        struct {                  // phase 3's elementwise part onwards
            float dlg[kC][kN];    // decay-gradient terms of each token
            float dkk[kC][kN];    // dKp * Kp (belongs to the previous token's decay)
            short outg[4][kC][kSK];  // dr, dk, da, dkappa (bf16), tokens x keys
        } e;
    } u;
    short rr[kC][kSK], kk[kC][kSK], ka[kC][kSK], aa[kC][kSK], ww[kC][kSK];  // raw inputs
    float gam[kC][kN];       // cumulative decay within the chunk
    float dlgc[8][kN];       // exit-state term: partial sums (4 value blocks, 4 token groups)
    float carry[4][kN];
};

// input (r, w, k, v, kappa, a, dy = 0..6) of the 128-piece row `slot` of a
// chunk's loads; a float32 decay is loaded apart, so its rows skip w
template <bool W32> __device__ constexpr int slot_input(int slot) {
    return (W32 && slot >= 1) ? (slot + 1 < 7 ? slot + 1 : 6) : (slot < 7 ? slot : 6);
}

template <bool W32>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void bwd_grad_kernel(
    BackwardArgs p) {
    __shared__ GradLds L;
    const int wave = threadIdx.x >> 6;
    const int nch = (p.T + kC - 1) / kC;
    const int ngrp = (nch + kGradChunks - 1) / kGradChunks;
    const long bh = blockIdx.x / ngrp;
    const int grp = (int)(blockIdx.x % ngrp);
    const int c_begin = grp * kGradChunks;
    const int c_end = min(nch, c_begin + kGradChunks);
    const long b = bh / p.H;
    const int h = (int)(bh % p.H);
    const uint16_t *in[7] = {static_cast<const uint16_t *>(p.r), static_cast<const uint16_t *>(p.w),
                             static_cast<const uint16_t *>(p.k), static_cast<const uint16_t *>(p.v),
                             static_cast<const uint16_t *>(p.kappa), static_cast<const uint16_t *>(p.a),
                             static_cast<const uint16_t *>(p.dy)};

    // A chunk's global inputs, loaded one chunk ahead (the chunks of the group
    // are walked last to first): its entry state (rows 16 wave + lo, keys
    // 16jb + g4 + e), for the group's last chunk its dSh from the workspace
    // (same layout), and the raw inputs as
    // 16-byte row pieces, piece q = threadIdx.x + 256 i (i < 4):
    //  - bf16 decay: q < 7 * 128 is keys/values 8 (q & 7) .. +7 of token
    //    (q >> 3) & 15 of input q >> 7 (r, w, k, v, kappa, a, dy);
    //  - float32 decay: q < 6 * 128 likewise over r, k, v, kappa, a, dy, and
    //    q' = q - 768 is keys 4 (q' & 15) .. +3 of token q' >> 4 of w.
    constexpr int kPieces = W32 ? 8 * 128 : 7 * 128;
    static_assert(kThreads == 256 && kPieces > 3 * kThreads && kPieces <= 4 * kThreads,
                  "three whole row pieces per thread and a fourth, whole or partial");
    float4 S0n[4];
    uint2 Dhn[4];  // bf16 dSh
    uint4 rawn[4];
    auto load_chunk = [&](int cc, bool with_dsh) {
        // thread index opaque per call, as for the LDS addresses below: the
        // per-thread address parts are recomputed instead of held across the loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int g4l = 4 * ((tid & 63) >> 4);
        const long srowl = (long)(16 * (tid >> 6) + (tid & 15)) * kN;
        const float *s0p = p.s_ckpt + (bh * nch + cc) * (long)(kN * kN) + srowl;
        const uint16_t *dsp = p.ds_ws + (bh * ngrp + grp) * (long)(kN * kN);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            S0n[jb] = *reinterpret_cast<const float4 *>(s0p + 16 * jb + g4l);
            if (with_dsh)
                Dhn[jb] = *reinterpret_cast<const uint2 *>(dsp + dsh_tile_offset(tid >> 6, jb, tid & 63));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kThreads * i;
            // known per i (256 threads): pieces 0..2 are bf16 row pieces; piece 3
            // is the float32 decay's, or dy's for the first 128 threads
            if (W32 || i < 3 || q < kPieces) {
                if (!(W32 && i == 3)) {
                    // input q >> 7, one of two known per i (the float32 decay's
                    // row skips w): a select of two pointers, not an indexed array
                    const uint16_t *src = ((q >> 7) & 1) ? in[slot_input<W32>(2 * i + 1)]
                                                          : in[slot_input<W32>(2 * i)];
                    const long t = (long)cc * kC + ((q >> 3) & 15);
                    const long o = tok_off(p, b, h, t < p.T ? t : 0) + 8 * (q & 7);
                    rawn[i] = *reinterpret_cast<const uint4 *>(src + o);
                } else {
                    const int qq = q - 6 * 128;
                    const long t = (long)cc * kC + (qq >> 4);
                    const long o = tok_off(p, b, h, t < p.T ? t : 0) + 4 * (qq & 15);
                    rawn[i] = *reinterpret_cast<const uint4 *>(static_cast<const float *>(p.w) + o);
                }
            }
        }
    };
    // raw pieces into the LDS input tiles (tokens x keys/values); tokens past T
    // become neutral: w = 1, all else 0
    auto stage_chunk = [&](long t0s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = threadIdx.x + kThreads * i;
            if (W32 || i < 3 || q < kPieces) {
                if (!(W32 && i == 3)) {
                    const int s = ((q >> 7) & 1) ? slot_input<W32>(2 * i + 1)
                                                  : slot_input<W32>(2 * i);
                    const int t = (q >> 3) & 15, k0 = 8 * (q & 7);
                    uint4 x = rawn[i];
                    if (t0s + t >= p.T) {
                        const unsigned fill = s == 1 ? 0x3F803F80u : 0u;  // bf16 1.0 pairs
                        x = make_uint4(fill, fill, fill, fill);
                    }
                    short *dst = s == 0 ? &L.rr[t][k0] : s == 1 ? &L.ww[t][k0]
                               : s == 2 ? &L.kk[t][k0] : s == 3 ? &L.vv[t][k0]
                               : s == 4 ? &L.ka[t][k0] : s == 5 ? &L.aa[t][k0] : &L.dyy[t][k0];
                    reinterpret_cast<uint2 *>(dst)[0] = make_uint2(x.x, x.y);
                    reinterpret_cast<uint2 *>(dst)[1] = make_uint2(x.z, x.w);
                } else {
                    // float32 decay: staged in the decay-product tile, which phase 1
                    // then overwrites element by element with the products
                    const int qq = q - 6 * 128, t = qq >> 4, k0 = 4 * (qq & 15);
                    uint4 x = rawn[i];
                    if (t0s + t >= p.T) x = make_uint4(0x3F800000u, 0x3F800000u, 0x3F800000u,
                                                       0x3F800000u);  // 1.0f
                    *reinterpret_cast<uint4 *>(&L.gam[t][k0]) = x;
                }
            }
        }
    };
    load_chunk(c_end - 1, true);
    // The state cotangent in fp32, in the layout of the dSh^T tiles: the group's
    // last chunk starts from its stored dSh; after each chunk's phase 2 it holds
    // that chunk's dS0, the earlier chunk's dS_C, whose dSh is it times the
    // earlier chunk's decay total per key (applied after that chunk's phase 1)
    f32x4 Dhf[4];
    __builtin_amdgcn_s_waitcnt(kWaitAllLoads);
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        const bf16x4 d = __builtin_bit_cast(bf16x4, Dhn[jb]);
        Dhf[jb] = f32x4{fbf(d[0]), fbf(d[1]), fbf(d[2]), fbf(d[3])};
    }

    for (int c = c_end - 1; c >= c_begin; --c) {
        // the lane index, opaque to the compiler in each iteration: otherwise every
        // LDS fragment address derived from it is hoisted out of the loop and held
        // in registers for the whole loop
        int lane_op = threadIdx.x & 63;
        asm volatile("" : "+v"(lane_op));
        const int lane = lane_op, lo = lane & 15, g4 = 4 * (lane >> 4);
        const long t0 = (long)c * kC;
        // outputs: element offset of the chunk's first token and the token stride;
        // every chunk but a ragged last one stores all 16 tokens without a test
        const long tb = tok_off(p, b, h, t0), TS = (long)p.H * kN;
        const bool full = t0 + kC <= p.T;
        f32x4 S0[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) S0[jb] = f32x4{S0n[jb].x, S0n[jb].y, S0n[jb].z, S0n[jb].w};

        // ---- phase 1: operands.  Thread (wave, lane): tokens 4 wave .. +3, key/value `lane`
        stage_chunk(t0);
        __syncthreads();
        {
            float x[7][4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * wave + e;
                x[0][e] = fbf(L.rr[t][lane]);
                x[1][e] = W32 ? L.gam[t][lane] : fbf(L.ww[t][lane]);  // w
                x[2][e] = fbf(L.kk[t][lane]);
                x[4][e] = fbf(L.ka[t][lane]); x[5][e] = fbf(L.aa[t][lane]);
            }
            float cp[4];
            cp[0] = x[1][0];
#pragma unroll
            for (int e = 1; e < 4; ++e) cp[e] = cp[e - 1] * x[1][e];
            L.carry[wave][lane] = cp[3];
            __syncthreads();
            float pre = 1.f;
#pragma unroll
            for (int q = 0; q < 4; ++q) pre = q < wave ? pre * L.carry[q][lane] : pre;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * wave + e;
                const float gam = pre * cp[e], gprev = e ? pre * cp[e - 1] : pre;
                const float r = x[0][e], k = x[2][e], kap = x[4][e], a = x[5][e];
                const float ig = __builtin_amdgcn_rcpf(gam);
                const float Kp = kap * gprev, Rp = r * gam, Km = k * ig, Bm = a * kap * ig;
                L.gam[t][lane] = gam;
                L.kp[t][lane] = bf1(Kp);
                L.rp[t][lane] = bf1(Rp);
                L.km[t][lane] = bf1(Km);
                L.bm[t][lane] = bf1(Bm);
            }
            __syncthreads();
        }
        if (c != c_end - 1) {
            // dSh = dS_C diag(g_C) with dS_C the later chunk's dS0
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const float4 gc = *reinterpret_cast<const float4 *>(&L.gam[kC - 1][16 * jb + g4]);
                Dhf[jb] = f32x4{Dhf[jb][0] * gc.x, Dhf[jb][1] * gc.y, Dhf[jb][2] * gc.z,
                                Dhf[jb][3] * gc.w};
            }
        }
        bf16x4 Dh[4];  // dSh as the bf16 MFMA operand
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) Dh[jb] = bf4(Dhf[jb]);

        // ---- chunk matrices, one share per wave, left in LDS as the bf16 A
        // operands every wave reads (wave 0: X = (I + N)^-1 and X^T from N = M_bk;
        // wave 1: M_kk, M_kk^T; wave 2: M_kr; wave 3: M_br).  They sit in the
        // state tiles' LDS, written only later in phase 2, hence the second
        // barrier.  (Every wave forming all of them, as it once did, was 45% of
        // the kernel's matrix-core products; a separate 4 KiB region would leave
        // two workgroups per CU instead of three and was slower.)
        bf16x4 (*fr)[64] = reinterpret_cast<bf16x4 (*)[64]>(&L.u);
        if (wave == 0) {
            Acc16 dn = z4(), dnt = z4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x4 kpa = frag(L.kp, 0, 16 * kb, lane), bma = frag(L.bm, 0, 16 * kb, lane);
                dn = mma(kpa, bma, dn);
                dnt = mma(bma, kpa, dnt);
            }
            dn = mask<true, true>(dn, lane);
            dnt = mask<false, true>(dnt, lane);
            f32x4 dx, dxt;  // D(X) = A operand of X^T, D(X^T) = A operand of X
            tri_inverse(dn.v, dnt.v, lane, dx, dxt);
            fr[0][lane] = bf4(dx);
            fr[1][lane] = bf4(dxt);
        } else if (wave == 1) {
            Acc16 m = z4(), mt = z4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x4 kpa = frag(L.kp, 0, 16 * kb, lane), kma = frag(L.km, 0, 16 * kb, lane);
                m = mma(kpa, kma, m);
                mt = mma(kma, kpa, mt);
            }
            fr[2][lane] = bf4(mask<true, true>(m, lane));
            fr[3][lane] = bf4(mask<false, true>(mt, lane));
        } else {
            const short(*rhs)[kSK] = wave == 2 ? L.km : L.bm;
            Acc16 m = z4();
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                m = mma(frag(L.rp, 0, 16 * kb, lane), frag(rhs, 0, 16 * kb, lane), m);
            fr[2 + wave][lane] = bf4(mask<true, false>(m, lane));
        }
        // the next chunk's inputs, in flight during the rest of this chunk
        if (c > c_begin) load_chunk(c - 1, false);
        __syncthreads();
        const bf16x4 fx = fr[0][lane], fxt = fr[1][lane], fmkk = fr[2][lane];
        const bf16x4 fmkkt = fr[3][lane], fmkr = fr[4][lane], fmbr = fr[5][lane];
        __syncthreads();  // phase 2 writes over the fragments

        // ---- phase 2: value block `wave` (tokens x values 16 wave ..)
        bf16x4 dvb;  // this lane's dv (tokens g4 .. g4+3, value 16 wave + lo)
        {
            // exit-state term sum_i dSh S0 over this block's values
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * jb + g4 + e;
                    const float s = sum_lanes16(Dhf[jb][e] * S0[jb][e]);
                    if (lo == 0) L.dlgc[wave][j] = s;
                    L.u.m.s0t[j][16 * wave + lo] = bf1(S0[jb][e]);
                    L.u.m.dsht[j][16 * wave + lo] = Dh[jb][e];
                }
            }
            const bf16x4 vb = colfrag(L.vv, 16 * wave, lane);    // B operand of V
            const bf16x4 dyb = colfrag(L.dyy, 16 * wave, lane);  // B operand of dY
            Acc16 z = mma(fmkkt, vb, z4());                      // Mkk V
            Acc16 du = mma(fmbr, dyb, z4());                     // Mbr^T dY
            Acc16 dv = mma(fmkr, dyb, z4());                     // Mkr^T dY
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const bf16x4 s0b = bf4(S0[jb]), dhb = Dh[jb];  // B operands of S0^T, dSh^T
                z = mma(frag(L.kp, 0, 16 * jb, lane), s0b, z);      // + Kp S0^T
                du = mma(frag(L.bm, 0, 16 * jb, lane), dhb, du);    // + Bm dSh^T
                dv = mma(frag(L.km, 0, 16 * jb, lane), dhb, dv);    // + Km dSh^T
            }
            du = neg(du);
            const Acc16 u = mma(fxt, bf4(z), z4());   // U = X Z
            const Acc16 dz = mma(fx, bf4(du), z4());  // dZ = X^T dU
            dv = mma(fmkk, bf4(dz), dv);              // + Mkk^T dZ
            // the chunk's entry cotangent dS0 = dSh + dY^T Rp + dZ^T Kp (as dS0^T
            // tiles: keys 16jb .., values 16 wave ..), the next chunk's dS_C
            if (c > c_begin) {
                const bf16x4 dzb = bf4(dz);
#pragma unroll
                for (int jb = 0; jb < 4; ++jb) {
                    Acc16 t = mma(colfrag(L.rp, 16 * jb, lane), dyb, Acc16{Dhf[jb]});
                    t = mma(colfrag(L.kp, 16 * jb, lane), dzb, t);
                    Dhf[jb] = t.v;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = g4 + e;
                L.uu[t][16 * wave + lo] = bf1(u[e]);
                L.dzz[t][16 * wave + lo] = bf1(dz[e]);
            }
            dvb = bf4(dv);  // stored with the other gradients after phase 3
        }
        __syncthreads();

        // ---- phase 3: key block `wave` (tokens x keys 16 wave ..)
        {
            // this wave's share of the chunk's cotangent matrices (wave 0: dMkr =
            // dY V^T and its transpose; wave 1: -dMbr = dY U^T; wave 2: dMkk = dZ V^T;
            // wave 3: -dMbk = dZ U^T), and the products with the state tiles
            Acc16 m0 = z4(), m1 = z4();
            Acc16 dkms = z4(), dbms = z4(), drp = z4(), dkp = z4();   // V dSh, U dSh, dY S0, dZ S0
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                const bf16x4 ya = frag(L.dyy, 0, 16 * vb, lane), va = frag(L.vv, 0, 16 * vb, lane);
                const bf16x4 ua = frag(L.uu, 0, 16 * vb, lane), za = frag(L.dzz, 0, 16 * vb, lane);
                const bf16x4 lhs = wave < 2 ? ya : za, rhs = (wave & 1) ? ua : va;
                m0 = mma(lhs, rhs, m0);
                m1 = mma(rhs, lhs, m1);
                const bf16x4 dsb = frag(L.u.m.dsht, 16 * wave, 16 * vb, lane);  // B operand of dSh
                const bf16x4 s0b = frag(L.u.m.s0t, 16 * wave, 16 * vb, lane);   // B operand of S0
                dkms = mma(va, dsb, dkms);
                dbms = mma(ua, dsb, dbms);
                drp = mma(ya, s0b, drp);
                dkp = mma(za, s0b, dkp);
            }
            // dMkr, -dMbr keep s <= t; dMkk, -dMbk s < t
            const bool strict = wave >= 2;
            __syncthreads();  // the state tiles are read: the fragments go over them
            fr[2 * wave][lane] = bf4(mask_rt<true>(m0, lane, strict));
            fr[2 * wave + 1][lane] = bf4(mask_rt<false>(m1, lane, strict));
            __syncthreads();
            const bf16x4 fdmr = fr[0][lane], fdmrt = fr[1][lane], fdmb = fr[2][lane];
            const bf16x4 fdmbt = fr[3][lane], fdmk = fr[4][lane], fdmkt = fr[5][lane];
            const bf16x4 fdmn = fr[6][lane], fdmnt = fr[7][lane];
            // Same-token parts of the decay terms below: the diagonals of dMkr and
            // dMbr and the first sub-diagonals of dMkk and dMbk enter one token's
            // dlg twice with opposite signs (through dRp and dKm, dBm, or dKm, dBm
            // and the next token's dKp), which cancel exactly, but only up to bf16
            // rounding once formed from differently rounded operands; dlg is taken
            // without them.  Wave 0 keeps them (as the products rounded them) in
            // the carry tile, free after phase 1: row k of 16 tokens.
            float *dg = &L.carry[0][0];
            if (wave == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = g4 + e;  // lane holds rows g4 .. g4+3 of column lo
                    if (row == lo) {
                        dg[0 * kC + lo] = fbf(fdmrt[e]);  // dMkr[t][t], as dRp took it
                        dg[1 * kC + lo] = fbf(fdmbt[e]);  // -dMbr[t][t], as dRp took it
                        dg[2 * kC + lo] = fbf(fdmr[e]);   // dMkr[t][t], as dKm took it
                        dg[3 * kC + lo] = fbf(fdmb[e]);   // -dMbr[t][t], as dBm took it
                    }
                    if (row == lo + 1) {
                        dg[4 * kC + lo] = fbf(fdmk[e]);   // dMkk[t+1][t] (dKm)
                        dg[5 * kC + lo] = fbf(fdmn[e]);   // -dMbk[t+1][t] (dBm)
                    }
                    if (row + 1 == lo) {
                        dg[6 * kC + lo] = fbf(fdmkt[e]);  // dMkk[t][t-1] (dKp)
                        dg[7 * kC + lo] = fbf(fdmnt[e]);  // -dMbk[t][t-1] (dKp)
                    }
                }
                if (lane == 0) {  // no token 16 or -1
                    dg[4 * kC + kC - 1] = 0.f;
                    dg[5 * kC + kC - 1] = 0.f;
                    dg[6 * kC] = 0.f;
                    dg[7 * kC] = 0.f;
                }
            }
            const bf16x4 rpb = colfrag(L.rp, 16 * wave, lane), kpb = colfrag(L.kp, 16 * wave, lane);
            const bf16x4 kmb = colfrag(L.km, 16 * wave, lane), bmb = colfrag(L.bm, 16 * wave, lane);
            // dKm = V dSh + dMkr^T Rp + dMkk^T Kp
            Acc16 dkm = mma(fdmk, kpb, mma(fdmr, rpb, dkms));
            // dBm = -U dSh - (-dMbr)^T Rp - (-dMbk)^T Kp
            Acc16 dbm = mma(fdmn, kpb, mma(fdmb, rpb, dbms));
            dbm = neg(dbm);
            // dRp = dY S0 + dMkr Km + dMbr Bm
            drp = mma(fdmrt, kmb, drp);
            drp = mma(negb(fdmbt), bmb, drp);
            // dKp = dZ S0 + dMkk Km + dMbk Bm
            dkp = mma(fdmkt, kmb, dkp);
            dkp = mma(negb(fdmnt), bmb, dkp);
            __syncthreads();  // the state tiles are read: their LDS is reused below
            // (and the value tiles: dv waits in U's)
#pragma unroll
            for (int e = 0; e < 4; ++e) L.uu[g4 + e][16 * wave + lo] = dvb[e];

            // elementwise: lane (token g4 + e, key 16 wave + lo)
            const int j = 16 * wave + lo;
            float csum = 0.f;
            float o_dr[4], o_dk[4], o_da[4], o_dkap[4];
            float4 sd[8];  // the same-token parts of tokens g4 .. g4+3
#pragma unroll
            for (int q = 0; q < 8; ++q) sd[q] = *reinterpret_cast<const float4 *>(&dg[q * kC + g4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = g4 + e;
                const float sA = (&sd[0].x)[e], sB = (&sd[1].x)[e], sC = (&sd[2].x)[e];
                const float sD = (&sd[3].x)[e], sE = (&sd[4].x)[e], sF = (&sd[5].x)[e];
                const float sG = (&sd[6].x)[e], sH = (&sd[7].x)[e];
                // the bf16 operands the products took
                const float bKm = fbf(L.km[t][j]), bRp = fbf(L.rp[t][j]), bBm = fbf(L.bm[t][j]);
                const int tn = t < kC - 1 ? t + 1 : t, tp = t ? t - 1 : t;
                const float bKpn = t < kC - 1 ? fbf(L.kp[tn][j]) : 0.f;
                const float bKmp = fbf(L.km[tp][j]), bBmp = fbf(L.bm[tp][j]);  // (0 weights at t = 0)
                const float gam = L.gam[t][j], gprev = t ? L.gam[t - 1][j] : 1.f;
                const float r = fbf(L.rr[t][j]), k = fbf(L.kk[t][j]), kap = fbf(L.ka[t][j]);
                const float a = fbf(L.aa[t][j]);
                const float ig = __builtin_amdgcn_rcpf(gam);
                const float Kp = kap * gprev, Rp = r * gam, Km = k * ig, Bm = a * kap * ig;
                const float dr = drp[e] * gam, dk = dkm[e] * ig, db = dbm[e] * ig;
                const float da = db * kap, dkap = dkp[e] * gprev + db * a;
                const float drp_d = drp[e] - sA * bKm + sB * bBm;
                const float dkm_d = dkm[e] - sC * bRp - sE * bKpn;
                const float dbm_d = dbm[e] + sD * bRp + sF * bKpn;
                const float dkp_d = dkp[e] - sG * bKmp + sH * bBmp;
                L.u.e.dlg[t][j] = drp_d * Rp - dkm_d * Km - dbm_d * Bm;
                L.u.e.dkk[t][j] = dkp_d * Kp;
                csum += Km * dkms[e] - Bm * dbms[e];  // exit-state term (dBm_S = -U dSh)
                o_dr[e] = dr; o_dk[e] = dk; o_da[e] = da; o_dkap[e] = dkap;
            }
            L.dlgc[4 + (lane >> 4)][j] = csum;
            // the gradients go out through LDS: stored from here, each store
            // instruction would write sixteen 32-byte pieces of token rows
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = g4 + e;
                L.u.e.outg[0][t][j] = bf1(o_dr[e]);
                L.u.e.outg[1][t][j] = bf1(o_dk[e]);
                L.u.e.outg[2][t][j] = bf1(o_da[e]);
                L.u.e.outg[3][t][j] = bf1(o_dkap[e]);
            }
        }
        __syncthreads();

        // ---- the chunk's dr, dk, da, dkappa and dv as whole token rows: wave q
        // stores tokens 4q .. 4q+3, four keys (values) per lane
        {
            const int tok = 4 * wave + (lane >> 4), k0 = 4 * lo;
            if (full || t0 + tok < p.T) {
                void *const dst[4] = {p.dr, p.dk, p.da, p.dkappa};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(dst[q]) + tb + tok * TS + k0) =
                        *reinterpret_cast<const uint2 *>(&L.u.e.outg[q][tok][k0]);
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.dv) + tb + tok * TS + k0) =
                    *reinterpret_cast<const uint2 *>(&L.uu[tok][k0]);
            }
        }

        // ---- phase 4: decay gradients, a reverse sum over the chunk's tokens per key
        if (wave == 0) {
            const int j = lane;
            // every LDS value first, then the sums
            // (float32 decay: w_t = g_t / g_{t-1} from the decay products, whose
            // tile held the raw w until phase 1)
            float dl[kC], dkn[kC], wv[kC], part[8];
#pragma unroll
            for (int t = 0; t < kC; ++t) {
                dl[t] = L.u.e.dlg[t][j];
                dkn[t] = L.u.e.dkk[t][j];
                wv[t] = W32 ? L.gam[t][j] : fbf(L.ww[t][j]);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) part[q] = L.dlgc[q][j];
            float acc = ((part[0] + part[1]) + (part[2] + part[3])) +
                        ((part[4] + part[5]) + (part[6] + part[7]));
            float dwv[kC];
#pragma unroll
            for (int t = kC - 1; t >= 0; --t) {
                acc += dl[t] + (t + 1 < kC ? dkn[t + 1] : 0.f);
                dwv[t] = W32 ? acc * (t ? wv[t - 1] : 1.f) * __builtin_amdgcn_rcpf(wv[t])
                             : acc * __builtin_amdgcn_rcpf(wv[t]);
            }
            if constexpr (W32) {
                float *q = static_cast<float *>(p.dw) + tb + j;
#pragma unroll
                for (int t = 0; t < kC; ++t)
                    if (full || t0 + t < p.T) q[t * TS] = dwv[t];
            } else {
                uint16_t *q = static_cast<uint16_t *>(p.dw) + tb + j;
                if (full) {
#pragma unroll
                    for (int t = 0; t < kC; ++t) q[t * TS] = bf1u(dwv[t]);
                } else {
#pragma unroll
                    for (int t = 0; t < kC; ++t)
                        if (t0 + t < p.T) q[t * TS] = bf1u(dwv[t]);
                }
            }
        }
        __syncthreads();  // the next chunk's operands overwrite LDS
    }
}

}  // namespace

size_t backward_chunked_workspace_bytes(int B, int T, int H) {
    const size_t nch = (size_t)(T + kC - 1) / kC;
    const size_t ngrp = (nch + kGradChunks - 1) / kGradChunks;
    return (size_t)B * H * ngrp * kN * kN * sizeof(uint16_t);
}

bool backward_chunked_grid_ok(int B, int T, int H) {
    const long heads = (long)B * H;
    const long ngrp = ((long)(T + kC - 1) / kC + kGradChunks - 1) / kGradChunks;
    return heads <= 0x7fffffffL && heads * ngrp <= 0x7fffffffL;
}

hipError_t launch_backward_chunked(const BackwardArgs &p, hipStream_t stream) {
    const long heads = (long)p.B * p.H;
    const long nch = (p.T + kC - 1) / kC;
    const long ngrp = (nch + kGradChunks - 1) / kGradChunks;
    if (p.w32) {
        hipLaunchKernelGGL(bwd_chain_kernel<true>, dim3((unsigned)heads), dim3(kChainThreads), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(bwd_grad_kernel<true>, dim3((unsigned)(heads * ngrp)), dim3(kThreads),
                           0, stream, p);
    } else {
        hipLaunchKernelGGL(bwd_chain_kernel<false>, dim3((unsigned)heads), dim3(kChainThreads), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(bwd_grad_kernel<false>, dim3((unsigned)(heads * ngrp)), dim3(kThreads),
                           0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace wkv7
