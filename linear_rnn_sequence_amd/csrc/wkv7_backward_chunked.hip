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
//   Mkr = tril(Rp Km^T), Mbr = tril(Rp Bm^T); X = (I + N)^-1;
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
//    like the forward chunked kernel's state); it stores each chunk's dSh in
//    bf16 (the MFMA operand both kernels use) to the workspace and writes ds0;
//  - bwd_grad_kernel: the chunks are independent here: from a chunk's stored
//    entry state and dSh a workgroup recomputes its operands and
//    forms every gradient; each workgroup takes 8 consecutive chunks of one
//    head and loads the next chunk's inputs while it works on the current one.
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

namespace wkv7 {
namespace {

typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kC = 16;        // tokens per chunk (the checkpoint interval)
constexpr int kThreads = 256;  // four waves
constexpr int kSK = 68;       // row stride (bf16) of 16 x 64 and 64 x 64 tiles
constexpr int kST = 20;       // row stride (bf16) of 64 x 16 (transposed) tiles
constexpr int kGradChunks = 8;  // consecutive chunks of one head per gradient workgroup

static_assert(kC == kCkpt, "chunks are the checkpoint intervals");

__device__ __forceinline__ f32x4 mma(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// two floats -> packed bf16 pair, round to nearest even (a vector conversion, so
// the compiler inserts the wait states an MFMA result needs before a VALU read)
__device__ __forceinline__ unsigned cvt2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ bf16x4 bf4(f32x4 x) {
    const u32x2 v = {cvt2(x[0], x[1]), cvt2(x[2], x[3])};
    return __builtin_bit_cast(bf16x4, v);
}
// one float -> bf16 bits, round to nearest even (the same hardware conversion)
__device__ __forceinline__ short bf1(float x) { return (short)(cvt2(x, 0.f) & 0xffffu); }
__device__ __forceinline__ uint16_t bf1u(float x) { return (uint16_t)(cvt2(x, 0.f) & 0xffffu); }
__device__ __forceinline__ float fbf(short s) { return __uint_as_float(((uint32_t)(uint16_t)s) << 16); }
__device__ __forceinline__ f32x4 z4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 neg(f32x4 x) { return f32x4{-x[0], -x[1], -x[2], -x[3]}; }

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
__device__ __forceinline__ f32x4 mask(f32x4 d, int lane) {
    const int lo = lane & 15, row = 4 * (lane >> 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = row + e;
        const bool keep = kLower ? (kStrict ? lo < r : lo <= r) : (kStrict ? r < lo : r <= lo);
        d[e] = keep ? d[e] : 0.f;
    }
    return d;
}

// D(((I + M)^-1)^T) for a nilpotent 16 x 16 M given dm = D(M), dmt = D(M^T):
// (I + M)^-1 = (I - M)(I + M^2)(I + M^4)(I + M^8), evaluated transposed as
//   F^T = (I - M^T) + (M^2)^T (I - M^T),  G^T = F^T + (M^4)^T F^T,
//   X^T = G^T + (M^8)^T G^T.
// Called with (D(N), D(N^T)) it gives D(X^T) = A operand of X; with the
// arguments swapped it gives D(X) = A operand of X^T.
__device__ __forceinline__ f32x4 inverse_t(f32x4 dm, f32x4 dmt, int lane) {
    const int lo = lane & 15, row = 4 * (lane >> 4);
    f32x4 imt;
#pragma unroll
    for (int e = 0; e < 4; ++e) imt[e] = (row + e == lo ? 1.f : 0.f) - dmt[e];
    const bf16x4 Mb = bf4(dm), Ma = bf4(dmt);
    const f32x4 m2 = mma(Ma, Mb, z4());   // D(M^2)
    const f32x4 m2t = mma(Mb, Ma, z4());  // D((M^2)^T)
    const bf16x4 M2b = bf4(m2), M2a = bf4(m2t);
    const f32x4 m4 = mma(M2a, M2b, z4());   // D(M^4)
    const f32x4 m4t = mma(M2b, M2a, z4());  // D((M^4)^T)
    const f32x4 ft = mma(M2b, bf4(imt), imt);  // D(F^T)
    const bf16x4 M4b = bf4(m4);
    const f32x4 gt = mma(M4b, bf4(ft), ft);    // D(G^T)
    const f32x4 m8 = mma(bf4(m4t), M4b, z4()); // D(M^8)
    return mma(bf4(m8), bf4(gt), gt);          // D(X^T)
}

// the decay's element type: bf16 bits, or float32 (RWKV7_DT_BF16_W32)
template <bool W32> struct DecayT { using type = uint16_t; };
template <> struct DecayT<true> { using type = float; };
__device__ __forceinline__ float widen(uint16_t u) { return bf16_lo(u); }
__device__ __forceinline__ float widen(float x) { return x; }

// Element offset of token t of (b, h) in a [B,T,H,64] tensor.
__device__ __forceinline__ long tok_off(const BackwardArgs &p, long b, int h, long t) {
    return ((b * p.T + t) * p.H + h) * kN;
}

// ---------------------------------------------------------------- reverse chain
struct ChainLds {
    short kp[kC][kSK], rp[kC][kSK], bm[kC][kSK];  // tokens x keys
    short dyy[kC][kSK];                           // tokens x values
    float carry[4][kN];                           // decay product of each wave's 4 tokens
    float gc[kN];                                 // decay total of the chunk
};

template <bool W32>
__global__ __launch_bounds__(kThreads) void bwd_chain_kernel(BackwardArgs p) {
    using WT = typename DecayT<W32>::type;
    __shared__ ChainLds L;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lo = lane & 15, g4 = 4 * (lane >> 4);
    const long bh = blockIdx.x;
    const long b = bh / p.H;
    const int h = (int)(bh % p.H);
    const int nch = (p.T + kC - 1) / kC;
    const uint16_t *pr = static_cast<const uint16_t *>(p.r);
    const WT *pw = static_cast<const WT *>(p.w);
    const uint16_t *pkap = static_cast<const uint16_t *>(p.kappa), *pa = static_cast<const uint16_t *>(p.a);
    const uint16_t *pdy = static_cast<const uint16_t *>(p.dy);

    // dS^T tiles: St[jb] holds dS^T[16jb + g4 + e][16 wave + lo] = dS[16 wave + lo][16jb + g4 + e]
    f32x4 St[4];
    const long srow = (long)(16 * wave + lo) * kN;
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
        if (p.ds_T) {
            const float4 x = *reinterpret_cast<const float4 *>(p.ds_T + bh * kN * kN + srow + 16 * jb + g4);
            St[jb] = f32x4{x.x, x.y, x.z, x.w};
        } else {
            St[jb] = z4();
        }
    }

    // raw bf16 inputs of a chunk: thread (wave, lane) takes key/value `lane` of
    // tokens 4 wave .. 4 wave + 3; the next chunk's are loaded while this one runs
    WT nw[4];
    uint16_t nk[4], na[4], nr[4], nd[4];
    auto load_chunk = [&](int cc) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const long t = (long)cc * kC + 4 * wave + e;
            const long o = tok_off(p, b, h, t < p.T ? t : 0) + lane;
            nw[e] = pw[o]; nk[e] = pkap[o]; na[e] = pa[o]; nr[e] = pr[o]; nd[e] = pdy[o];
        }
    };
    load_chunk(nch - 1);

    for (int c = nch - 1; c >= 0; --c) {
        float wv[4], kv[4], av[4], rv[4], dv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = (long)c * kC + 4 * wave + e < p.T;
            wv[e] = ok ? widen(nw[e]) : 1.f;
            kv[e] = ok ? bf16_lo(nk[e]) : 0.f;
            av[e] = ok ? bf16_lo(na[e]) : 0.f;
            rv[e] = ok ? bf16_lo(nr[e]) : 0.f;
            dv[e] = ok ? bf16_lo(nd[e]) : 0.f;
        }
        if (c > 0) load_chunk(c - 1);
        float cp[4];
        cp[0] = wv[0];
#pragma unroll
        for (int e = 1; e < 4; ++e) cp[e] = cp[e - 1] * wv[e];
        L.carry[wave][lane] = cp[3];
        __syncthreads();
        float pre = 1.f, tot = 1.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float x = L.carry[q][lane];
            pre = q < wave ? pre * x : pre;
            tot *= x;
        }
        if (wave == 0) L.gc[lane] = tot;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 4 * wave + e;
            const float gam = pre * cp[e], gprev = e ? pre * cp[e - 1] : pre;
            const float Kp = kv[e] * gprev, Rp = rv[e] * gam;
            const float Bm = av[e] * kv[e] * __builtin_amdgcn_rcpf(gam);
            L.kp[t][lane] = bf1(Kp);
            L.rp[t][lane] = bf1(Rp);
            L.bm[t][lane] = bf1(Bm);
            L.dyy[t][lane] = bf1(dv[e]);
        }
        __syncthreads();

        // ---- chunk matrices (every wave forms its own copy)
        f32x4 dn = z4(), dnt = z4(), dmbr = z4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x4 kpa = frag(L.kp, 0, 16 * kb, lane), bma = frag(L.bm, 0, 16 * kb, lane);
            const bf16x4 rpa = frag(L.rp, 0, 16 * kb, lane);
            dn = mma(kpa, bma, dn);     // D(N), N = Kp Bm^T
            dnt = mma(bma, kpa, dnt);   // D(N^T)
            dmbr = mma(rpa, bma, dmbr); // D(Mbr), Mbr = Rp Bm^T
        }
        dn = mask<true, true>(dn, lane);
        dnt = mask<false, true>(dnt, lane);
        dmbr = mask<true, false>(dmbr, lane);
        const f32x4 dx = inverse_t(dnt, dn, lane);  // D(X) = A operand of X^T

        // ---- chain step: dSh = dS_C diag(g_C), stored as the bf16 MFMA operand
        // that both kernels use, then dS0 of the chunk
        uint16_t *ck = p.ds_ws + (bh * nch + c) * (long)(kN * kN) + srow;
        bf16x4 Sb[4];
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) St[jb][e] *= L.gc[16 * jb + g4 + e];
            Sb[jb] = bf4(St[jb]);  // B operand of dSh^T (keys x values)
            *reinterpret_cast<bf16x4 *>(ck + 16 * jb + g4) = Sb[jb];
        }
        const bf16x4 dyb = colfrag(L.dyy, 16 * wave, lane);  // B operand of dY (tokens x values)
        f32x4 rhs = mma(bf4(dmbr), dyb, z4());                // Mbr^T dY
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) rhs = mma(frag(L.bm, 0, 16 * jb, lane), Sb[jb], rhs);  // + Bm dSh^T
        const f32x4 up = mma(bf4(dx), bf4(rhs), z4());  // X^T rhs = -dZ
        const bf16x4 dzb = bf4(neg(up));
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            St[jb] = mma(colfrag(L.rp, 16 * jb, lane), dyb, St[jb]);  // + Rp^T dY (A of Rp^T)
            St[jb] = mma(colfrag(L.kp, 16 * jb, lane), dzb, St[jb]);  // + Kp^T dZ
        }
        __syncthreads();  // the next chunk's operands overwrite LDS
    }
    if (p.ds0) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            *reinterpret_cast<float4 *>(p.ds0 + bh * kN * kN + srow + 16 * jb + g4) =
                make_float4(St[jb][0], St[jb][1], St[jb][2], St[jb][3]);
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
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lo = lane & 15, g4 = 4 * (lane >> 4);
    const int nch = (p.T + kC - 1) / kC;
    const int ngrp = (nch + kGradChunks - 1) / kGradChunks;
    const long bh = blockIdx.x / ngrp;
    const int c_begin = (int)(blockIdx.x % ngrp) * kGradChunks;
    const int c_end = min(nch, c_begin + kGradChunks);
    const long b = bh / p.H;
    const int h = (int)(bh % p.H);
    const uint16_t *in[7] = {static_cast<const uint16_t *>(p.r), static_cast<const uint16_t *>(p.w),
                             static_cast<const uint16_t *>(p.k), static_cast<const uint16_t *>(p.v),
                             static_cast<const uint16_t *>(p.kappa), static_cast<const uint16_t *>(p.a),
                             static_cast<const uint16_t *>(p.dy)};

    // A chunk's global inputs, loaded one chunk ahead: its entry state and dSh
    // (rows 16 wave + lo, keys 16jb + g4 + e) and the raw inputs as
    // 16-byte row pieces, piece q = threadIdx.x + 256 i (i < 4):
    //  - bf16 decay: q < 7 * 128 is keys/values 8 (q & 7) .. +7 of token
    //    (q >> 3) & 15 of input q >> 7 (r, w, k, v, kappa, a, dy);
    //  - float32 decay: q < 6 * 128 likewise over r, k, v, kappa, a, dy, and
    //    q' = q - 768 is keys 4 (q' & 15) .. +3 of token q' >> 4 of w.
    constexpr int kPieces = W32 ? 8 * 128 : 7 * 128;
    static_assert(kThreads == 256 && kPieces > 3 * kThreads && kPieces <= 4 * kThreads,
                  "three whole row pieces per thread and a fourth, whole or partial");
    const long srow = (long)(16 * wave + lo) * kN;
    float4 S0n[4];
    uint2 Dhn[4];  // bf16 dSh
    uint4 rawn[4];
    auto load_chunk = [&](int cc) {
        // thread index opaque per call, as for the LDS addresses below: the
        // per-thread address parts are recomputed instead of held across the loop
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int g4l = 4 * ((tid & 63) >> 4);
        const long srowl = (long)(16 * (tid >> 6) + (tid & 15)) * kN;
        const float *s0p = p.s_ckpt + (bh * nch + cc) * (long)(kN * kN) + srowl;
        const uint16_t *dsp = p.ds_ws + (bh * nch + cc) * (long)(kN * kN) + srowl;
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            S0n[jb] = *reinterpret_cast<const float4 *>(s0p + 16 * jb + g4l);
            Dhn[jb] = *reinterpret_cast<const uint2 *>(dsp + 16 * jb + g4l);
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
    load_chunk(c_begin);

    for (int c = c_begin; c < c_end; ++c) {
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
        auto put4 = [&](void *base, long off, const float (&x)[4]) {  // tokens g4 .. g4+3
            uint16_t *q = static_cast<uint16_t *>(base) + tb + off;
            if (full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) q[(g4 + e) * TS] = bf1u(x[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (t0 + g4 + e < p.T) q[(g4 + e) * TS] = bf1u(x[e]);
            }
        };
        f32x4 S0[4];
        bf16x4 Dh[4];  // dSh, bf16 as stored
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            S0[jb] = f32x4{S0n[jb].x, S0n[jb].y, S0n[jb].z, S0n[jb].w};
            Dh[jb] = __builtin_bit_cast(bf16x4, Dhn[jb]);
        }

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
        if (c + 1 < c_end) load_chunk(c + 1);  // in flight during the rest of this chunk

        // ---- chunk matrices (every wave forms its own copy)
        f32x4 dmkk = z4(), dmkkt = z4(), dn = z4(), dnt = z4(), dmkr = z4(), dmbr = z4();
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x4 kpa = frag(L.kp, 0, 16 * kb, lane), kma = frag(L.km, 0, 16 * kb, lane);
            const bf16x4 bma = frag(L.bm, 0, 16 * kb, lane), rpa = frag(L.rp, 0, 16 * kb, lane);
            dmkk = mma(kpa, kma, dmkk);
            dmkkt = mma(kma, kpa, dmkkt);
            dn = mma(kpa, bma, dn);
            dnt = mma(bma, kpa, dnt);
            dmkr = mma(rpa, kma, dmkr);
            dmbr = mma(rpa, bma, dmbr);
        }
        dmkk = mask<true, true>(dmkk, lane);
        dmkkt = mask<false, true>(dmkkt, lane);
        dn = mask<true, true>(dn, lane);
        dnt = mask<false, true>(dnt, lane);
        dmkr = mask<true, false>(dmkr, lane);
        dmbr = mask<true, false>(dmbr, lane);
        const f32x4 dxt = inverse_t(dn, dnt, lane);  // D(X^T) = A operand of X
        const f32x4 dx = inverse_t(dnt, dn, lane);   // D(X)   = A operand of X^T

        // ---- phase 2: value block `wave` (tokens x values 16 wave ..)
        {
            // exit-state term sum_i dSh S0 over this block's values
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * jb + g4 + e;
                    const float s = sum_lanes16(fbf(Dh[jb][e]) * S0[jb][e]);
                    if (lo == 0) L.dlgc[wave][j] = s;
                    L.u.m.s0t[j][16 * wave + lo] = bf1(S0[jb][e]);
                    L.u.m.dsht[j][16 * wave + lo] = Dh[jb][e];
                }
            }
            const bf16x4 vb = colfrag(L.vv, 16 * wave, lane);    // B operand of V
            const bf16x4 dyb = colfrag(L.dyy, 16 * wave, lane);  // B operand of dY
            f32x4 z = mma(bf4(dmkkt), vb, z4());                 // Mkk V
            f32x4 du = mma(bf4(dmbr), dyb, z4());                // Mbr^T dY
            f32x4 dv = mma(bf4(dmkr), dyb, z4());                // Mkr^T dY
#pragma unroll
            for (int jb = 0; jb < 4; ++jb) {
                const bf16x4 s0b = bf4(S0[jb]), dhb = Dh[jb];  // B operands of S0^T, dSh^T
                z = mma(frag(L.kp, 0, 16 * jb, lane), s0b, z);      // + Kp S0^T
                du = mma(frag(L.bm, 0, 16 * jb, lane), dhb, du);    // + Bm dSh^T
                dv = mma(frag(L.km, 0, 16 * jb, lane), dhb, dv);    // + Km dSh^T
            }
            du = neg(du);
            const f32x4 u = mma(bf4(dxt), bf4(z), z4());   // U = X Z
            const f32x4 dz = mma(bf4(dx), bf4(du), z4());  // dZ = X^T dU
            dv = mma(bf4(dmkk), bf4(dz), dv);              // + Mkk^T dZ
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = g4 + e;
                L.uu[t][16 * wave + lo] = bf1(u[e]);
                L.dzz[t][16 * wave + lo] = bf1(dz[e]);
            }
            const float dvv[4] = {dv[0], dv[1], dv[2], dv[3]};
            put4(p.dv, 16 * wave + lo, dvv);
        }
        __syncthreads();

        // ---- phase 3: key block `wave` (tokens x keys 16 wave ..)
        {
            f32x4 dmr = z4(), dmrt = z4(), dmb = z4(), dmbt = z4();   // dMkr, dMkr^T, -dMbr, -dMbr^T
            f32x4 dmk = z4(), dmkt = z4(), dmn = z4(), dmnt = z4();   // dMkk, dMkk^T, -dMbk, -dMbk^T
            f32x4 dkms = z4(), dbms = z4(), drp = z4(), dkp = z4();   // V dSh, U dSh, dY S0, dZ S0
#pragma unroll
            for (int vb = 0; vb < 4; ++vb) {
                const bf16x4 ya = frag(L.dyy, 0, 16 * vb, lane), va = frag(L.vv, 0, 16 * vb, lane);
                const bf16x4 ua = frag(L.uu, 0, 16 * vb, lane), za = frag(L.dzz, 0, 16 * vb, lane);
                dmr = mma(ya, va, dmr);
                dmrt = mma(va, ya, dmrt);
                dmb = mma(ya, ua, dmb);
                dmbt = mma(ua, ya, dmbt);
                dmk = mma(za, va, dmk);
                dmkt = mma(va, za, dmkt);
                dmn = mma(za, ua, dmn);
                dmnt = mma(ua, za, dmnt);
                const bf16x4 dsb = frag(L.u.m.dsht, 16 * wave, 16 * vb, lane);  // B operand of dSh
                const bf16x4 s0b = frag(L.u.m.s0t, 16 * wave, 16 * vb, lane);   // B operand of S0
                dkms = mma(va, dsb, dkms);
                dbms = mma(ua, dsb, dbms);
                drp = mma(ya, s0b, drp);
                dkp = mma(za, s0b, dkp);
            }
            dmr = mask<true, false>(dmr, lane);
            dmrt = mask<false, false>(dmrt, lane);
            dmb = mask<true, false>(dmb, lane);
            dmbt = mask<false, false>(dmbt, lane);
            dmk = mask<true, true>(dmk, lane);
            dmkt = mask<false, true>(dmkt, lane);
            dmn = mask<true, true>(dmn, lane);
            dmnt = mask<false, true>(dmnt, lane);
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
                        dg[0 * kC + lo] = fbf(bf1(dmrt[e]));  // dMkr[t][t], as dRp took it
                        dg[1 * kC + lo] = fbf(bf1(dmbt[e]));  // -dMbr[t][t], as dRp took it
                        dg[2 * kC + lo] = fbf(bf1(dmr[e]));   // dMkr[t][t], as dKm took it
                        dg[3 * kC + lo] = fbf(bf1(dmb[e]));   // -dMbr[t][t], as dBm took it
                    }
                    if (row == lo + 1) {
                        dg[4 * kC + lo] = fbf(bf1(dmk[e]));   // dMkk[t+1][t] (dKm)
                        dg[5 * kC + lo] = fbf(bf1(dmn[e]));   // -dMbk[t+1][t] (dBm)
                    }
                    if (row + 1 == lo) {
                        dg[6 * kC + lo] = fbf(bf1(dmkt[e]));  // dMkk[t][t-1] (dKp)
                        dg[7 * kC + lo] = fbf(bf1(dmnt[e]));  // -dMbk[t][t-1] (dKp)
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
            f32x4 dkm = mma(bf4(dmk), kpb, mma(bf4(dmr), rpb, dkms));
            // dBm = -U dSh - (-dMbr)^T Rp - (-dMbk)^T Kp
            f32x4 dbm = mma(bf4(dmn), kpb, mma(bf4(dmb), rpb, dbms));
            dbm = neg(dbm);
            // dRp = dY S0 + dMkr Km + dMbr Bm
            drp = mma(bf4(dmrt), kmb, drp);
            drp = mma(bf4(neg(dmbt)), bmb, drp);
            // dKp = dZ S0 + dMkk Km + dMbk Bm
            dkp = mma(bf4(dmkt), kmb, dkp);
            dkp = mma(bf4(neg(dmnt)), bmb, dkp);
            __syncthreads();  // the state tiles are read: their LDS is reused below

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
            put4(p.dr, j, o_dr);
            put4(p.dk, j, o_dk);
            put4(p.da, j, o_da);
            put4(p.dkappa, j, o_dkap);
        }
        __syncthreads();

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
    return (size_t)B * H * nch * kN * kN * sizeof(uint16_t);
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
        hipLaunchKernelGGL(bwd_chain_kernel<true>, dim3((unsigned)heads), dim3(kThreads), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(bwd_grad_kernel<true>, dim3((unsigned)(heads * ngrp)), dim3(kThreads),
                           0, stream, p);
    } else {
        hipLaunchKernelGGL(bwd_chain_kernel<false>, dim3((unsigned)heads), dim3(kThreads), 0,
                           stream, p);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(bwd_grad_kernel<false>, dim3((unsigned)(heads * ngrp)), dim3(kThreads),
                           0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace wkv7
