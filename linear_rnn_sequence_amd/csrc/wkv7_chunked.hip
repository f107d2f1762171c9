// WKV7 chunked-parallel prefill (ALGO_CHUNKED) on bf16 MFMA with a float32
// state carried between chunks.
//
// The pages state that the transition is diagonal plus rank one and that this
// keeps the recurrence parallelisable in chunks (RWKV-7 "Goose" summary, §4
// Method, "efficient computation"; §8 Speed and Memory, chunked pre-fill), and
// that a chunked bf16 kernel exists (author response on numerical precision),
// but they give no algorithm.  The form used here follows from the update
//   S_t = S_{t-1} diag(w_t) - u_t b_t^T + v_t k_t^T,  u_t = S_{t-1} kappa_t,
//   b_t = a_t * kappa_t,  y_t = S_t r_t
// (author response, numpy time_mixing listing) by unrolling it over a chunk of
// C = 16 tokens with entry state S0.  With G_t = prod_{s<=t} w_s (G_{-1} = 1):
//   Kp_t = kappa_t * G_{t-1}   Rp_t = r_t * G_t   Km_s = k_s / G_s   Bm_s = b_s / G_s
//   M_kk[t,s] = Kp_t.Km_s (s<t)   M_bk[t,s] = Kp_t.Bm_s (s<t)
//   M_kr[t,s] = Rp_t.Km_s (s<=t)  M_br[t,s] = Rp_t.Bm_s (s<=t)
//   U   = (I + M_bk)^-1 (Kp S0^T + M_kk V)        (rows: the u_t of the chunk)
//   Y   = Rp S0^T + M_kr V - M_br U
//   S_C^T = diag(G_C) (S0^T + Km^T V - Bm^T U)
// (the last line is diag(G_C) S0^T plus the writes and removals decayed by
// G_C / G_s; summing before the scaling keeps every term's relative error at
// fp32 level because the scaled result is a sum of terms of ordinary size).
// The kernel carries U' = -U (it stores -(I + M_bk)^-1) so no other operand
// needs a sign flip.
// Every product is a 16 x 16 bf16 MFMA with fp32 accumulation (pairs of K = 16
// products as one v_mfma_f32_16x16x32_bf16); the state stays fp32 in the
// accumulators.  The unit lower-triangular inverse (I + M_bk)^-1 is formed by
// block substitution (tri_inverse in wkv7_mfma.h: float32 4 x 4 diagonal
// blocks, then float32 matrix-core products), so it stays accurate when
// removal keys repeat or correlate within a chunk.  The decay ratios stay
// within w_min^-16 (1.6e4 for the pages' w > 0.545).  Requires 0 < w <= 1.
//
// Work split: one workgroup of 8 waves per (batch, head), walking the chunks
// in order as a three-stage pipeline with one barrier per chunk:
//   waves 4..7 ("prep"): wave 4+b prepares tokens 4b .. 4b+3 of chunk c+2
//     (one token per DPP row, its 64 keys over the row's 16 lanes, so loads
//     read whole token rows) from raw inputs held 4 chunks deep in a register
//     ring, writes the chunk's bf16 operand tiles to LDS, and forms one C x C
//     matrix of chunk c+1 (wave 5: the triangular inverse).  The decay
//     prefix over the chunk is a scan over each wave's four rows plus the
//     earlier waves' totals, left in LDS one interval ahead;
//   waves 0..3 ("chain"): wave b owns value block i in [16b, 16b+16) of the
//     state: S^T is held as four 16x16 fp32 accumulator tiles per wave, in
//     exactly the layout the next chunk's MFMAs consume, so the state never
//     leaves registers; they run chunk c's MFMA chain and finish chunk c-1's
//     readouts (GroupNorm statistics need all four value blocks).
// A SIMD thus holds one chain wave and one prep wave; LDS holds the operands
// of three chunks (81,760 bytes, so two workgroups fit on a CU), each MFMA
// operand pair stored side by side per row so that a lane reads both halves
// of a 16x16x32 operand with one 16-byte LDS read.  Alone on a CU an
// interval is bound by the inverse wave; with two workgroups, by instruction
// issue on the SIMDs (the prep waves run at a raised wave priority).
//
// Wait counts: vector stores count with loads on this target, so a full wait
// inside the chunk loop would also wait for the chunk's stores.  Loads made
// before the loop are waited for once before it, optional loads are
// branch-free and consumed in the iteration that issues them (or carried raw
// to the next one), and the prep ring states its own wait count.
//
// Variants (template parameters and ForwardArgs fields):
//   - segments: long sequences of few heads are cut into parallel time
//     segments; a summary pass computes each segment's transition (state
//     started at I, v = 0) and offset (started at 0), each chain wave carrying
//     both for its value rows (the same eight waves, so two workgroups still
//     share a CU), a combine kernel
//     forms the entry states S_in[g+1] = S_in[g] P_g + dS_g in fp32, and the
//     main pass reruns every segment from its entry state;
//   - W32: the decay arrives as float32;
//   - FUSED: raw keys in, kappa = normalise(k * k_k) and k + k (a-1) k_a formed
//     in the prep lanes, output gate applied to the finished readouts;
//   - reverse / y_f32 / YADD: the two passes of the bidirectional forward (a
//     negative token stride; float32 readouts out; added readouts in);
//   - s_ckpt: the training forward stores the state entering every chunk.
//
// MFMA 16x16x16 bf16 lane layouts (lane l, g = l / 16, e = 0..3; the
// 16x16x32 form holds 8 consecutive k per lane in both A and B):
//   A[m][k]: lane holds A[l%16][4g+e];  B[k][n]: lane holds B[4g+e][l%16];
//   D[m][n]: lane holds D[4g+e][l%16].
// So a D tile is directly a B operand, and the A form of X is the B form of X^T.
#include "wkv7_device.h"
#include "wkv7_internal.h"
#include "wkv7_mfma.h"

namespace wkv7 {

const bool kChunkedAvailable = true;

namespace {

constexpr int kC = 16;                  // tokens per chunk
constexpr int kPrefetch = 4;            // chunks of raw inputs in flight per lane
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] + vmcnt[15:14], expcnt[6:4],
// lgkmcnt[11:8]); expcnt and lgkmcnt are left unlimited.  wait_older_chunks
// lets the (kPrefetch-1) youngest chunks' loads stay in flight: vmcnt = loads
// per chunk x (kPrefetch-1), six loads per chunk (r, w, k, kappa, a, v), five
// with the fused prologue (no kappa).
constexpr int kWaitAllLoads = (0x7 << 4) | (0xF << 8);  // vmcnt(0) only
constexpr int kUnroll = 2 * kPrefetch;                   // prep loop unroll

// Whether this workgroup holds an odd slot on its CU: the thread-group ID field
// of the HW_ID hardware register (bits 19:16; s_getreg operand = register 4,
// offset 16, width 4).  Of two workgroups placed on one CU the first gets
// slot 0 and the second slot 1.
__device__ __forceinline__ bool workgroup_slot_odd() {
    return (__builtin_amdgcn_s_getreg(4 | (16 << 6) | (3 << 11)) & 1u) != 0;
}

// Intervals 0 .. S-1 of the prep waves' loop: the nch chunks rounded up to
// whole loop trips.  In all, the prep waves run max(nch + 3, S) intervals and
// the chain waves match them.
__device__ __forceinline__ int steady_intervals(int nch) {
    return (nch + kUnroll - 1) / kUnroll * kUnroll;
}

constexpr int wait_older_chunks(int loads_per_chunk) {
    return ((loads_per_chunk * (kPrefetch - 1)) & 0xF) | (0x7 << 4) | (0xF << 8) |
           ((((loads_per_chunk * (kPrefetch - 1)) >> 4) & 0x3) << 14);
}
// Head-size geometry (NH = 64 or 128 keys and values per head): one chain wave
// per 16-value block; prep waves in groups of four, each group preparing 64 of
// every token's keys.
template <int NH>
struct Geo {
    static constexpr int KB = NH / 16;      // key blocks (= value blocks = chain waves)
    static constexpr int KH = NH / 64;      // prep groups
    static constexpr int CW = KB;           // chain waves
    static constexpr int PW = 4 * KH;       // prep waves
    static constexpr int threads = 64 * (CW + PW);
};
constexpr int kThreads = Geo<64>::threads;  // 4 chain waves + 4 prep waves
constexpr int kThreadsMW = kThreads + 64;   // ... and a matrix wave
constexpr int kRow = 20;                // bf16 per LDS tile row (16 + 4 pad, 40 bytes)
constexpr int kTile = 16 * kRow;        // bf16 per 16x16 tile
// A pair tile holds two 16x16 tiles (X | Y) so that a lane's K = 32 operand
// (X's four k beside Y's four) is 16 contiguous bytes: row r, column c of half
// h at r * kPRow + (c / 4) * 8 + 4h + c % 4 (80-byte rows: the 16-byte reads
// of eight lanes of one column group hit disjoint banks).
constexpr int kPRow = 40;
constexpr int kPTile = 16 * kPRow;
// Distances between the tiles of one array (16 rows plus padding) chosen so
// that the prep waves' stores (a lane writes one token of four keys; the
// transposed tiles take them as 2-byte stores down a column) and the chain
// waves' reads spread over the LDS banks: with the bare tile sizes the key
// blocks of one store instruction all met in the same banks (up to 8-way).
constexpr int kPTileRows = 672;  // Kp, Rp, Km, Bm pair tiles
constexpr int kPTileCols = 648;  // (Km^T | Bm^T) pair tiles
constexpr int kTileVt = 324;     // V^T tiles
constexpr int kTileVr = 336;     // V row tiles

template <int NH>
struct __align__(16) ChunkOps {
    // pair tiles over key blocks (2p | 2p+1), rows t (or s), columns j
    short kp[NH / 32][kPTileRows];  // Kp  (A form rows t; also B form of Kp^T)
    short rp[NH / 32][kPTileRows];  // Rp
    short km[NH / 32][kPTileRows];  // Km
    short bm[NH / 32][kPTileRows];  // Bm
    short kbt[NH / 16][kPTileCols]; // (Km^T | Bm^T) of key block jb: rows j, columns s
    short mkz[kPTile];     // (M_kk | 0)  [t][s]; the zero half is set once
    short mrb[kPTile];     // (M_kr | M_br)  [t][s]
    short xinv[kTile];     // -(I + M_bk)^-1 [t][s]
    short vt[NH / 16][kTileVt];  // V^T [value block][i][t]  (B form of V)
    short vr[NH / 16][kTileVr];  // V   [value block][t][i]  (epilogue only)
    float gc[NH];          // G_C per key j
    // per token sums over each prep group's 64 keys, fp32: [0] r_t.k_t,
    // [1] r_t.(a_t*kappa_t), [2] the bonus sum_j r k r_k
    float rsum[NH / 64][3][16];
    // the sum over all keys of token t, quantity q
    __device__ __forceinline__ float rsum_all(int q, int t) const {
        float x = rsum[0][q][t];
#pragma unroll
        for (int h = 1; h < NH / 64; ++h) x += rsum[h][q][t];
        return x;
    }
};

// Launch description: the sequence may be split into nseg segments of seg_len
// tokens (the last one shorter) that are processed in parallel; the workspace
// holds per (b, h, segment) the transition P, the offset dS and the entry state.
struct ChunkedParams {
    ForwardArgs p;
    int nseg;         // segments per sequence
    int nseg_launch;  // segments per (b, h) covered by this launch
    int seg_len;      // tokens per segment (a multiple of kC)
    float *ws_p, *ws_ds, *ws_sin;
};

template <int NH>
struct __align__(16) ChunkSmem {
    ChunkOps<NH> ops[3];
    float2 stats[2][16][NH / 16];  // per token, per value block: (mean, M2) of 16 readouts
    // per prep group and chunk parity, reading prep wave r and slot b < 3: the
    // product of w over prep wave b's four tokens if b < r, else 1 (set once), so
    // a reader multiplies its three slots without selects
    float4 carry[NH / 64][2][4][3][16];
};

// lane's K = 32 operand of a pair tile (A form of X | Y side by side)
__device__ __forceinline__ bf16x8s ld_pair(const short *ptile, int lane) {
    return *reinterpret_cast<const bf16x8s *>(ptile + (lane & 15) * kPRow + 8 * (lane >> 4));
}
// lane's A-form values of half h of a pair tile
__device__ __forceinline__ void st_pair(short *ptile, int h, int lane, bf16x4 x) {
    *reinterpret_cast<bf16x4 *>(ptile + (lane & 15) * kPRow + 8 * (lane >> 4) + 4 * h) = x;
}
__device__ __forceinline__ bf16x4 ld_a(const short *tile, int lane) {
    return *reinterpret_cast<const bf16x4 *>(tile + (lane & 15) * kRow + 4 * (lane >> 4));
}
__device__ __forceinline__ void st_a(short *tile, int lane, bf16x4 x) {
    *reinterpret_cast<bf16x4 *>(tile + (lane & 15) * kRow + 4 * (lane >> 4)) = x;
}

// Raw inputs of one chunk held by one lane: token t = lane % 16 of the chunk,
// channels 16w + 4g .. +3 of each of the six vectors (keys for r, w, k, kappa,
// a; values for v).  W32: the decay arrives as float32.
template <bool W32>
struct RawW {
    using T = uint2;  // four bf16
};
template <>
struct RawW<true> {
    using T = float4;
};
template <bool W32>
struct Raw {
    uint2 r, k, kap, a, v;  // kap unused with the fused prologue
    typename RawW<W32>::T w;
};

// Fused prologue parameters of a prep lane: k_k and k_a of its four channels.
struct ProParams {
    float kk[4];
    float ka[4];
};

// Who forms a chunk's triangular inverse (Chunked::matrices)
constexpr int kMatInPrep = 0;  // prep wave 1 of group 0, after its other work
constexpr int kMatSplit = 1;   // a matrix wave of its own; the prep waves skip it
constexpr int kMatWave = 2;    // the matrix wave itself

template <bool EPI, bool W32, bool FUSED, int NH>
struct Chunked {
    static_assert(!FUSED || NH == 64, "the fused prologue is built for head size 64");
    using Ops = ChunkOps<NH>;
    const ForwardArgs &p;
    // blk: value block (chain waves) or prep wave within its group; kh: prep group
    // (keys 64kh .. 64kh+63 of every token)
    const int lane, blk, kh, g, lo;
    const int Tl;                // tokens of this workgroup's range
    // Elements from one token to the next in processing order (negative when the
    // sequence is walked from its end), and the offset of (b, token t0 of the
    // processing order, h, 0).
    const long TS, tok0;
    const long lane_off;  // prep lane: its token (ptok) of chunk 0, keys 64kh + 4lo .. +3

    __device__ Chunked(const ForwardArgs &p_, int b_, int h_, int t0, int tl, int blk_, int kh_)
        : p(p_), lane(threadIdx.x & 63), blk(blk_), kh(kh_),
          g((threadIdx.x & 63) >> 4), lo(threadIdx.x & 15), Tl(tl),
          TS(p_.reverse ? -(long)p_.H * NH : (long)p_.H * NH),
          tok0(((long)b_ * p_.T + (p_.reverse ? p_.T - 1 - t0 : t0)) * ((long)p_.H * NH) +
               (long)h_ * NH),
          lane_off(tok0 + (long)(4 * blk_ + ((threadIdx.x & 63) >> 4)) * TS + 64 * kh_ +
                   4 * (threadIdx.x & 15)) {}

    // Prep lanes are token-major: prep wave b of group kh holds tokens 4b .. 4b+3
    // of a chunk, one per DPP row g, and lane lo of the row holds keys 64kh + 4lo
    // .. +3, so the row holds 64 consecutive keys of the token and each load
    // instruction reads four whole 128-byte rows (a key-block split would touch
    // sixteen partial lines).
    __device__ __forceinline__ int ptok() const { return 4 * blk + g; }

    // Issues the same loads on every path (no branch around them), so the
    // compiler's wait-count bookkeeping can leave the later chunks of the ring in
    // flight: the chunk index is clamped to the last chunk and the token index to
    // T-1, which keeps every address inside the tensors; unpack() replaces the
    // values of tokens past T.
    __device__ void load(int c, Raw<W32> &x) const {
        const int cc = min(c, (Tl - 1) / kC);
        const int t = min(cc * kC + ptok(), Tl - 1);
        const long off = lane_off + (long)(t - ptok()) * TS;
        x.r = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.r) + off);
        if constexpr (W32)
            x.w = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.w) + off);
        else
            x.w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.w) + off);
        x.k = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.k) + off);
        if constexpr (!FUSED)
            x.kap = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.kappa) + off);
        x.a = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.a) + off);
        x.v = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.v) + off);
    }

    // valid: the lane's token lies inside the range.  A padding token of a
    // partial last chunk (its loads were clamped to the last token) gets k = 0,
    // kappa = 0 and w = 1: no write, no removal and no decay, so it changes
    // neither the state nor any other token's readout (its own is not stored).
    // Selects rather than a branch: a branch that rewrites the prefetch ring's
    // registers turns the compiler's wait counts for the ring conservative.
    __device__ __forceinline__ void unpack_w(const Raw<W32> &x, bool valid, float (&w)[4]) const {
        if constexpr (W32) {
            w[0] = x.w.x; w[1] = x.w.y; w[2] = x.w.z; w[3] = x.w.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = valid ? w[e] : 1.f;
        } else {
            const unsigned w01 = valid ? x.w.x : 0x3F803F80u, w23 = valid ? x.w.y : 0x3F803F80u;
            w[0] = bf16_lo(w01); w[1] = bf16_hi(w01);
            w[2] = bf16_lo(w23); w[3] = bf16_hi(w23);
        }
    }

    // The raw inputs of one lane (its token, four keys) widened to float, kp =
    // kappa (with the fused prologue formed here from the raw keys).
    struct Unpacked {
        float r[4], k[4], a[4], kp[4];
        uint2 v;
    };
    __device__ Unpacked unpack(const Raw<W32> &x, bool valid, const ProParams &pro) const {
        Unpacked u;
        float *r = u.r, *k = u.k, *a = u.a, *kp = u.kp;
        r[0] = bf16_lo(x.r.x); r[1] = bf16_hi(x.r.x); r[2] = bf16_lo(x.r.y); r[3] = bf16_hi(x.r.y);
        const unsigned k01 = valid ? x.k.x : 0u, k23 = valid ? x.k.y : 0u;
        k[0] = bf16_lo(k01); k[1] = bf16_hi(k01); k[2] = bf16_lo(k23); k[3] = bf16_hi(k23);
        a[0] = bf16_lo(x.a.x); a[1] = bf16_hi(x.a.x); a[2] = bf16_lo(x.a.y); a[3] = bf16_hi(x.a.y);
        if constexpr (FUSED) {
            // kappa = normalise(k * k_k) over the token's 64 keys (the DPP row);
            // k <- k + k (a-1) k_a
            float kk[4], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kk[e] = k[e] * pro.kk[e];
                ss += kk[e] * kk[e];
            }
            ss = sum_lanes16(ss);
            const float inv = 1.f / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kp[e] = kk[e] * inv;
                k[e] = k[e] + k[e] * (a[e] - 1.f) * pro.ka[e];
            }
        } else {
            const unsigned c01 = valid ? x.kap.x : 0u, c23 = valid ? x.kap.y : 0u;
            kp[0] = bf16_lo(c01); kp[1] = bf16_hi(c01);
            kp[2] = bf16_lo(c23); kp[3] = bf16_hi(c23);
        }
        u.v = x.v;
        return u;
    }

    // Products of w over the prep wave's four tokens (the DPP rows g) for the
    // lane's four keys: lp inclusive, lx exclusive.  Row pairs by
    // v_permlane16_swap (even rows receive row g+1, odd rows row g-1), then the
    // pair (0, 1) total into rows 2, 3 by v_permlane32_swap (its first result
    // holds, in lanes 32..63, lanes 0..31 of the second operand).  Row 3's lp is
    // the wave's total, stored in the slots of the chunk's later prep waves.
    __device__ void scan(const float (&w)[4], float (&lp)[4], float (&lx)[4],
                         float4 (&slots)[4][3][16]) const {
        const bool odd = g & 1, upper = g >= 2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // the two results hold the lane's own value and its partner's in an
            // order that depends on the row, so the pair product uses both and
            // the own value needs no separate copy
            const auto h16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[e]),
                                                              __float_as_uint(w[e]), false, false);
            const float h0 = __uint_as_float(h16[0]), h1 = __uint_as_float(h16[1]);
            const float pair = h0 * h1;
            const float in1 = odd ? pair : h0;   // even rows: h0 is the own value
            const float ex1 = odd ? h0 : 1.f;    // odd rows: h0 is the row below
            const auto h32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair),
                                                              __float_as_uint(pair), false, false);
            const float below = upper ? __uint_as_float(h32[0]) : 1.f;
            lp[e] = in1 * below;
            lx[e] = ex1 * below;
        }
        if (g == 3) {
            const float4 t = make_float4(lp[0], lp[1], lp[2], lp[3]);
#pragma unroll
            for (int r = 1; r < 4; ++r)
                if (r > blk) slots[r][blk][lo] = t;
        }
    }

    // Chunk operands of the lane's token and keys, written to LDS buffer `o`.
    // lp, lx: the scan of this chunk; carry: this wave's slots of the chunk.
    // RD = false (the segment summary pass, no readouts): without Rp and the
    // diagonals of M_kr and M_br, which only the readouts use.
    template <bool RD>
    __device__ void prep(const Unpacked &u, Ops &o, const float (&rk)[4],
                         const float (&lp)[4], const float (&lx)[4],
                         const float4 (&carry)[3][16]) const {
        const float *r = u.r, *k = u.k, *a = u.a, *kp = u.kp;
        // decay of the chunk's tokens before this wave's four: the earlier waves'
        // totals (slots of later waves hold 1), read in one LDS round trip
        const float4 w0 = carry[0][lo], w1 = carry[1][lo], w2 = carry[2][lo];
        const float c[4] = {w0.x * w1.x * w2.x, w0.y * w1.y * w2.y, w0.z * w1.z * w2.z,
                            w0.w * w1.w * w2.w};
        f32x4 G, Kp, Rp, Km, Bm;
        float bon = 0.f, dkr = 0.f, dbr = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float q = c[e] * lp[e];               // G_t = prod_{s<=t} w_s
            G[e] = q;
            const float iG = __builtin_amdgcn_rcpf(q);  // 1 ulp; operands are rounded to bf16
            const float be = a[e] * kp[e];
            Kp[e] = kp[e] * (c[e] * lx[e]);             // kappa_t G_{t-1} (G_{-1} = 1)
            Km[e] = k[e] * iG;
            Bm[e] = be * iG;
            if constexpr (RD) {
                Rp[e] = r[e] * q;
                if (EPI) bon += r[e] * k[e] * rk[e];
                dkr += r[e] * k[e];
                dbr += r[e] * be;
            }
        }
        // the lane's 4 keys sit in key block jb at columns c0 .. c0+3: row t of
        // half jb % 2 of pair tile jb / 2
        const int t = ptok(), jb = 4 * kh + (lo >> 2), c0 = 4 * (lo & 3);
        const int rowoff = t * kRow + c0;
        const int poff = t * kPRow + 8 * (lo & 3) + 4 * (jb & 1);
        *reinterpret_cast<bf16x4 *>(o.kp[jb >> 1] + poff) = to_bf16(Kp);
        if constexpr (RD) *reinterpret_cast<bf16x4 *>(o.rp[jb >> 1] + poff) = to_bf16(Rp);
        const bf16x4 kmb = to_bf16(Km), bmb = to_bf16(Bm);
        *reinterpret_cast<bf16x4 *>(o.km[jb >> 1] + poff) = kmb;
        *reinterpret_cast<bf16x4 *>(o.bm[jb >> 1] + poff) = bmb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // transposed: row = key c0+e, column = token t
            const int toff = (c0 + e) * kPRow + 8 * (t >> 2) + (t & 3);
            o.kbt[jb][toff] = kmb[e];
            o.kbt[jb][toff + 4] = bmb[e];
        }
        if (EPI)  // V rows [t][i] for the bonus term of the readouts
            *reinterpret_cast<uint2 *>(o.vr[jb] + rowoff) = u.v;
        o.vt[jb][(c0 + 0) * kRow + t] = (short)(u.v.x & 0xffffu);
        o.vt[jb][(c0 + 1) * kRow + t] = (short)(u.v.x >> 16);
        o.vt[jb][(c0 + 2) * kRow + t] = (short)(u.v.y & 0xffffu);
        o.vt[jb][(c0 + 3) * kRow + t] = (short)(u.v.y >> 16);
        // the last token's lanes hold the whole-chunk decay G_C
        if (t == kC - 1) *reinterpret_cast<float4 *>(&o.gc[64 * kh + 4 * lo]) =
            make_float4(G[0], G[1], G[2], G[3]);
        // fp32 diagonals of M_kr and M_br: at s = t the decay ratio is exactly 1, so
        // r_t.k_t and r_t.(a_t*kappa_t) need no bf16 factors; the two-factor bf16
        // form would leave an absolute error of ~2^-9 sum_j |r_j k_j| that dominates
        // early readouts whose dot product nearly cancels.  Sums over the group's
        // 64 keys of the token: the 16 lanes of the DPP row.
        if constexpr (RD) {
            dkr = sum_lanes16(dkr);
            dbr = sum_lanes16(dbr);
            if (EPI) bon = sum_lanes16(bon);
            if (lo == 0) {
                o.rsum[kh][0][t] = dkr;
                o.rsum[kh][1][t] = dbr;
                if (EPI) o.rsum[kh][2][t] = bon;
            }
        }
    }

    // One C x C matrix of a chunk per prep wave of group 0 (contractions over all
    // NH keys); wave 1 of the group forms the triangular inverse.  RD = false:
    // M_kr and M_br (waves 2 and 3), which only the readouts use, are skipped.
    // MODE kMatInPrep: as above; kMatSplit: a prep wave whose workgroup has a
    // matrix wave (wave 1 forms nothing); kMatWave: the matrix wave, which forms
    // the inverse only.
    template <bool RD, int MODE>
    __device__ void matrices(Ops &o) const {
        const int row = 4 * g;  // D rows of this lane: row .. row+3; D column: lo
        if (MODE == kMatWave) {
            inverse(o);
            return;
        }
        if (kh != 0 || (!RD && blk >= 2)) return;
        if (blk == 1) {
            if (MODE == kMatInPrep) inverse(o);
        } else {
            // blk 0: M_kk^T = Km.Kp^T, strict; blk 2: M_kr^T = Km.Rp^T; blk 3: M_br^T
            const short(*lhs)[kPTileRows] = (blk == 3) ? o.bm : o.km;
            const short(*rhs)[kPTileRows] = (blk == 0) ? o.kp : o.rp;
            Acc32 am = Acc32::zero();
#pragma unroll
            for (int q = 0; q < NH / 32; ++q)
                am = mfma32(ld_pair(lhs[q], lane), ld_pair(rhs[q], lane), am);
            f32x4 m = am.v;
            // D[s = row+e][t = lo] = A form of M at [t = lo][s = row+e]
            const float diag = (blk != 0) ? o.rsum_all(blk == 2 ? 0 : 1, lo) : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool keep = (blk == 0) ? (row + e < lo) : (row + e <= lo);
                const float val = (blk != 0 && row + e == lo) ? diag : m[e];
                m[e] = keep ? val : 0.f;
            }
            st_pair(blk == 0 ? o.mkz : o.mrb, blk == 3 ? 1 : 0, lane, to_bf16(m));
        }
    }

    // -(I + M_bk)^-1 of a chunk into o.xinv (its A form, negated)
    __device__ void inverse(Ops &o) const {
        const int row = 4 * g;  // D rows of this lane: row .. row+3; D column: lo
        // D(M) below: the MFMA result layout of M (lane holds M[4g+e][lo]), which
        // is the B form of M and the A form of M^T.
        // N = M_bk (strictly lower): nb = D(N) from Kp.Bm^T, na = D(N^T) from Bm.Kp^T
        Acc32 anb = Acc32::zero(), ana = Acc32::zero();
#pragma unroll
        for (int q = 0; q < NH / 32; ++q) {
            const bf16x8s kpq = ld_pair(o.kp[q], lane), bmq = ld_pair(o.bm[q], lane);
            anb = mfma32(kpq, bmq, anb);
            ana = mfma32(bmq, kpq, ana);
        }
        f32x4 nb = anb.v, na = ana.v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            nb[e] = (lo < row + e) ? nb[e] : 0.f;   // [t = row+e][s = lo], s < t
            na[e] = (row + e < lo) ? na[e] : 0.f;   // [s = row+e][t = lo], s < t
        }
        f32x4 dx, dxt;
        tri_inverse(nb, na, lane, dx, dxt);
        st_a(o.xinv, lane, to_bf16(-dxt));  // A form of X = D(X^T), stored negated
    }
};

// Per-chain-lane state carried from chunk c's chain to its readout stores one
// interval later.  The chain forms Y^T, so lane (g, lo) of chain wave blk holds
// the readouts of token lo of the chunk at the four value channels
// i = 16blk + 4g + e: y[e], with v of the same token and channels, the token's
// bonus sum and (fused prologue) the raw bf16 output gates.
struct Pending {
    f32x4 y;
    float bon;
    uint2 graw;  // four bf16 gates
    uint2 v;     // four bf16 values
};

template <bool EPI, bool W32, bool FUSED, int NH>
__device__ __forceinline__ void finish_readouts(const ForwardArgs &p,
                                                const Chunked<EPI, W32, FUSED, NH> &K,
                                                const ChunkSmem<NH> &sm, const Pending &pd,
                                                int c, const float (&lnw)[4],
                                                const float (&lnb)[4], long yoff) {
    float yv[4] = {pd.y[0], pd.y[1], pd.y[2], pd.y[3]};
    if (EPI) {
        // GroupNorm statistics of this lane's token from the value blocks' (mean,
        // M2) (Chan et al. pairwise combination of equal-sized groups)
        constexpr int VB = NH / 16;
        const float4 *st = reinterpret_cast<const float4 *>(sm.stats[c & 1][K.lo]);
        float4 m[VB / 2];
        float ssum = 0.f, m2 = 0.f;
#pragma unroll
        for (int i = 0; i < VB / 2; ++i) {
            m[i] = st[i];
            ssum += m[i].x + m[i].z;
            m2 += m[i].y + m[i].w;
        }
        const float mu = ssum * (1.f / VB);
        float dev = 0.f;
#pragma unroll
        for (int i = 0; i < VB / 2; ++i) {
            const float d0 = m[i].x - mu, d1 = m[i].z - mu;
            dev += d0 * d0 + d1 * d1;
        }
        m2 += 16.f * dev;
        const float rs = __builtin_amdgcn_rsqf(m2 * (1.f / NH) + p.epi.eps);
        const float v[4] = {bf16_lo(pd.v.x), bf16_hi(pd.v.x), bf16_lo(pd.v.y), bf16_hi(pd.v.y)};
#pragma unroll
        for (int e = 0; e < 4; ++e) yv[e] = (yv[e] - mu) * (rs * lnw[e]) + lnb[e] + pd.bon * v[e];
    }
    if (FUSED && p.g) {  // output gate
        yv[0] *= bf16_lo(pd.graw.x);
        yv[1] *= bf16_hi(pd.graw.x);
        yv[2] *= bf16_lo(pd.graw.y);
        yv[3] *= bf16_hi(pd.graw.y);
    }
    // yoff: element offset of (token c*16 + lo, channel 16blk + 4g)
    if (c * kC + K.lo >= K.Tl) return;  // padding token of a partial last chunk
    if (p.y_f32) {  // float32 readouts, no rounding (first pass of a bidirectional call)
        *reinterpret_cast<float4 *>(p.y_f32 + yoff) = make_float4(yv[0], yv[1], yv[2], yv[3]);
        return;
    }
    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.y) + yoff) =
        make_uint2(cvt_pk(yv[0], yv[1]), cvt_pk(yv[2], yv[3]));
}

// SUMMARY = false: y and the final state of each (b, h, segment) from its entry
//   state (the whole sequence when there is one segment).
// SUMMARY = true: for each (b, h, segment) but the last, the segment's offset
//   dS (entry state 0) and transition P (entry state I, v = 0), both as final
//   states, both carried by chain wave b for value rows 16b .. 16b+15; no
//   readouts.  Final state = S_in P + dS.
// YADD: add the float32 readouts p.y_add (the reverse pass of a bidirectional
// call) before the epilogue.
//
// NH = 128 (head size 128): eight chain waves (one per value block) and two prep
// groups of four waves, each group preparing 64 of every token's keys; 1024
// threads.  No segments (one workgroup per CU already), no fused prologue, no
// bidirectional pass and no stored states.
template <bool EPI, bool SUMMARY, bool W32, bool FUSED, bool YADD, int NH, bool MW>
__global__ __launch_bounds__(Geo<NH>::threads + (MW ? 64 : 0))
__attribute__((amdgpu_waves_per_eu(MW ? 3 : 4))) void chunked_kernel(
    ChunkedParams cp) {
    static_assert(NH == 64 || (!SUMMARY && !YADD && !MW), "head size 128: plain forward only");
    using G = Geo<NH>;
    constexpr int KB = G::KB;
    __shared__ ChunkSmem<NH> sm;
    const ForwardArgs &p = cp.p;
    const int bh = blockIdx.x / cp.nseg_launch;
    const int seg = blockIdx.x - bh * cp.nseg_launch;
    const int b = bh / p.H, h = bh - b * p.H;
    const int t0 = seg * cp.seg_len;
    const int wave = threadIdx.x >> 6;
    // chain waves 0 .. CW-1; prep waves CW .. CW+PW-1 in groups of four
    const bool chain_wave = wave < G::CW;
    // MW: wave CW + PW forms each chunk's triangular inverse and nothing else (it
    // takes the place of prep wave 1 of group 0 in the inverse's index math)
    const bool matrix_wave = MW && wave == G::CW + G::PW;
    const int wblk = chain_wave ? (wave & (G::CW - 1)) : matrix_wave ? 1 : ((wave - G::CW) & 3);
    const int wkh = (chain_wave || matrix_wave) ? 0 : (wave - G::CW) >> 2;
    const Chunked<EPI, W32, FUSED, NH> K(p, b, h, t0, min(cp.seg_len, p.T - t0), wblk, wkh);
    const int lane = K.lane, blk = K.blk, g = K.g, lo = K.lo;
    const int nch = (K.Tl + kC - 1) / kC;
    constexpr long NN = (long)NH * NH;
    const long srow = (long)(16 * blk + lo) * NH;   // this lane's value row i in a state
    const long sidx = (long)bh * cp.nseg + seg;     // (b, h, segment) slot in the workspace
    // entry state and where the final state goes
    const float *s_in = SUMMARY ? nullptr
                      : (cp.nseg == 1 ? (p.s0 ? p.s0 + (long)bh * NN : nullptr)
                                      : cp.ws_sin + sidx * NN);
    float *s_fin = SUMMARY ? cp.ws_ds + sidx * NN
                 : (seg == cp.nseg - 1 && p.s_out ? p.s_out + (long)bh * NN : nullptr);
    // stored states (training forward): chunk c of this range is global chunk t0/kC + c
    static_assert(kC == kCkpt, "a chunk is one checkpoint interval");
    float *ckpt = (!SUMMARY && p.s_ckpt)
                      ? p.s_ckpt + ((long)bh * ((p.T + kC - 1) / kC) + t0 / kC) * NN
                      : nullptr;

    if (chain_wave) {
        // ---------------- chain waves: state, MFMA chain, readouts ----------------
        // S^T tile jb holds rows j = 16jb + 4g + e, column i = 16blk + lo.  SUMMARY:
        // Z is the offset (entry state 0) and Zp the transition (entry state I,
        // v = 0) of the same value rows, advanced side by side over the chunks.
        Acc32 Z[KB], Zp[KB];
#pragma unroll
        for (int jb = 0; jb < KB; ++jb) {
            if (s_in) {
                const float4 x = *reinterpret_cast<const float4 *>(s_in + srow + 16 * jb + 4 * g);
                Z[jb].v = f32x4{x.x, x.y, x.z, x.w};
            } else {
                Z[jb] = Acc32::zero();
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
                Zp[jb].v[e] = (16 * jb + 4 * g + e == 16 * blk + lo) ? 1.f : 0.f;
        }
        // GroupNorm weight and bias of this lane's four value channels
        float lnw[4] = {1.f, 1.f, 1.f, 1.f}, lnb[4] = {0.f, 0.f, 0.f, 0.f};
        const int ich = h * NH + 16 * blk + 4 * g;
        if (EPI && p.epi.ln_w) {
            const float4 q = *reinterpret_cast<const float4 *>(p.epi.ln_w + ich);
            lnw[0] = q.x; lnw[1] = q.y; lnw[2] = q.z; lnw[3] = q.w;
        }
        if (EPI && p.epi.ln_b) {
            const float4 q = *reinterpret_cast<const float4 *>(p.epi.ln_b + ich);
            lnb[0] = q.x; lnb[1] = q.y; lnb[2] = q.z; lnb[3] = q.w;
        }
        Pending pd;
        bf16x8s VU = {0, 0, 0, 0, 0, 0, 0, 0};  // (V | -U) of the chunk, as B operand
        bf16x8s VUp = {0, 0, 0, 0, 0, 0, 0, 0};  // SUMMARY: (0 | -U) of the transition
        // element offset of (token lo of the chunk, value channel 16blk + 4g)
        long ylane = K.tok0 + (long)lo * K.TS + 16 * blk + 4 * g;
        // added readouts of a chunk, loaded at the start of its iteration and used
        // after its MFMA chain (token index clamped into the range: no branch
        // around the loads, and no load waited for across the loop's back edge)
        constexpr bool kYadd = YADD && !SUMMARY;
        float4 ya = make_float4(0.f, 0.f, 0.f, 0.f);
        auto load_ya = [&](int cc) {
            ya = *reinterpret_cast<const float4 *>(
                p.y_add + K.tok0 + (long)min(cc * kC + lo, K.Tl - 1) * K.TS + 16 * blk + 4 * g);
        };
        // everything loaded so far is in registers before the chunk loop, so no
        // wait for these loads is left inside it
        __builtin_amdgcn_s_waitcnt(kWaitAllLoads);
        const long ystep = (long)kC * K.TS;
        auto store_state = [&](float *dst) {  // non-temporal: read back only by the backward
            // key tiles 2h and 2h+1 trade the halves of their rows between lanes lo
            // and lo ^ 8 (DPP row rotation by 8), so that each store writes 8 rows x
            // 128 bytes (whole lines) instead of 16 rows x 64 bytes
            const bool upper = lo >= 8;
            const int rA = 16 * blk + (upper ? lo - 8 : lo), rB = rA + 8;
#pragma unroll
            for (int h = 0; h < KB / 2; ++h) {
                f32x4 A, B;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ra = dpp_mov<kDppRowRor8>(Z[2 * h].v[e]);
                    const float rb = dpp_mov<kDppRowRor8>(Z[2 * h + 1].v[e]);
                    A[e] = upper ? rb : Z[2 * h].v[e];
                    B[e] = upper ? Z[2 * h + 1].v[e] : ra;
                }
                const int col = 32 * h + (upper ? 16 : 0) + 4 * g;
                __builtin_nontemporal_store(A, reinterpret_cast<f32x4 *>(dst + (long)rA * NH + col));
                __builtin_nontemporal_store(B, reinterpret_cast<f32x4 *>(dst + (long)rB * NH + col));
            }
        };
        if (ckpt && nch > 0) store_state(ckpt);  // the state before chunk 0
        __syncthreads();  // interval -1: decay totals of chunk 0
        __syncthreads();  // interval 0: chunk 0 prepared
        __syncthreads();  // interval 1: chunk 0 matrices, chunk 1 prepared
        for (int c = 0; c <= nch; ++c) {
            if (!SUMMARY && c > 0) {
                finish_readouts<EPI, W32, FUSED, NH>(p, K, sm, pd, c - 1, lnw, lnb, ylane);
                ylane += ystep;
            }
            if (c < nch) {
                if (kYadd) load_ya(c);  // the other direction's readouts of this chunk
                if (FUSED && !SUMMARY) {
                    // output gate of this chunk's readouts, loaded without branches (a
                    // branch around loads makes the compiler wait for all of them):
                    // the token index is clamped into the range and, without a gate,
                    // the raw keys (same shape) are read and the value discarded
                    // (the bits are only widened where the readouts are finished, one
                    // chunk later, so nothing waits for these loads before the barrier)
                    const uint16_t *gsrc = static_cast<const uint16_t *>(p.g ? p.g : p.k);
                    pd.graw = *reinterpret_cast<const uint2 *>(
                        gsrc + K.tok0 + (long)min(c * kC + lo, K.Tl - 1) * K.TS + 16 * blk + 4 * g);
                }
                const ChunkOps<NH> &o = sm.ops[c % 3];
                if constexpr (SUMMARY) {
                    // the offset's and the transition's chunk steps (independent,
                    // so the two dependent MFMA chains interleave); no readouts
                    auto advance = [&](Acc32(&Zs)[KB], bf16x8s & VUs) {
                        bf16x8s ZP[KB / 2];
#pragma unroll
                        for (int q = 0; q < KB / 2; ++q) {
                            ZP[q].lo = to_bf16(Zs[2 * q].v);
                            ZP[q].hi = to_bf16(Zs[2 * q + 1].v);
                        }
                        Acc32 rhs = mfma32(ld_pair(o.mkz, lane), VUs, Acc32::zero());
#pragma unroll
                        for (int q = 0; q < KB / 2; ++q)
                            rhs = mfma32(ld_pair(o.kp[q], lane), ZP[q], rhs);
                        const Acc16 U = mfma16(ld_a(o.xinv, lane), to_bf16(rhs.v), Acc16::zero());
                        VUs.hi = to_bf16(U.v);
#pragma unroll
                        for (int jb = 0; jb < KB; ++jb) {
                            Zs[jb] = mfma32(ld_pair(o.kbt[jb], lane), VUs, Zs[jb]);
                            const float4 gc = *reinterpret_cast<const float4 *>(&o.gc[16 * jb + 4 * g]);
                            Zs[jb].v[0] *= gc.x;
                            Zs[jb].v[1] *= gc.y;
                            Zs[jb].v[2] *= gc.z;
                            Zs[jb].v[3] *= gc.w;
                        }
                    };
                    VU.lo = ld_a(o.vt[blk], lane);
                    advance(Z, VU);
                    advance(Zp, VUp);  // (V | -U) with V = 0
                    __syncthreads();
                    continue;
                }
                // B operands as 8-wide pairs: (V | -U) and the state pairs; one K =
                // 32 MFMA per two 16-k products, accumulation chains within that
                // one opcode
                VU.lo = ld_a(o.vt[blk], lane);
                bf16x8s ZP[KB / 2];  // state pairs (key blocks 2q | 2q+1)
#pragma unroll
                for (int q = 0; q < KB / 2; ++q) {
                    ZP[q].lo = to_bf16(Z[2 * q].v);
                    ZP[q].hi = to_bf16(Z[2 * q + 1].v);
                }
                // rhs = M_kk V + Kp S0^T; (M_kk | 0) meets (V | the previous chunk's
                // -U), whose product with the zero half vanishes
                Acc32 rhs = mfma32(ld_pair(o.mkz, lane), VU, Acc32::zero());
#pragma unroll
                for (int q = 0; q < KB / 2; ++q) rhs = mfma32(ld_pair(o.kp[q], lane), ZP[q], rhs);
                // readouts as Y^T = S0 Rp^T + V^T M_kr^T - U^T M_br^T (the operands of
                // Y with their roles swapped): lane holds Y^T[i = 4g+e][t = lo]; the
                // terms without U first, so only one product waits for U
                Acc32 Y = Acc32::zero();
#pragma unroll
                for (int q = 0; q < KB / 2; ++q) Y = mfma32(ZP[q], ld_pair(o.rp[q], lane), Y);
                const Acc16 U = mfma16(ld_a(o.xinv, lane), to_bf16(rhs.v), Acc16::zero());  // -U
                VU.hi = to_bf16(U.v);
                Y = mfma32(VU, ld_pair(o.mrb, lane), Y);
#pragma unroll
                for (int jb = 0; jb < KB; ++jb) {
                    Z[jb] = mfma32(ld_pair(o.kbt[jb], lane), VU, Z[jb]);
                    const float4 gc = *reinterpret_cast<const float4 *>(&o.gc[16 * jb + 4 * g]);
                    Z[jb].v[0] *= gc.x;
                    Z[jb].v[1] *= gc.y;
                    Z[jb].v[2] *= gc.z;
                    Z[jb].v[3] *= gc.w;
                }
                if (kYadd) {  // (a padding token's sum is never stored)
                    Y.v[0] += ya.x;
                    Y.v[1] += ya.y;
                    Y.v[2] += ya.z;
                    Y.v[3] += ya.w;
                }
                pd.y = Y.v;
                // stored states: the one leaving this chunk enters the next; stored
                // here, in the slack before the barrier, rather than just before
                // the MFMAs that overwrite the accumulators
                if (ckpt && c + 1 < nch) store_state(ckpt + (long)(c + 1) * NN);
                if (EPI && !SUMMARY) {
                    pd.bon = o.rsum_all(2, lo);
                    pd.v = *reinterpret_cast<const uint2 *>(o.vr[blk] + lo * kRow + 4 * g);
                    // mean and M2 of token lo's readouts over this value block: four
                    // in the lane, summed over the four DPP rows g
                    const float mu = sum_rows4((Y[0] + Y[1]) + (Y[2] + Y[3])) * (1.f / 16.f);
                    const float d0 = Y[0] - mu, d1 = Y[1] - mu, d2 = Y[2] - mu, d3 = Y[3] - mu;
                    const float m2 = sum_rows4((d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3));
                    if (g == 0) sm.stats[c & 1][lo][blk] = make_float2(mu, m2);
                }
            }
            __syncthreads();
        }
        // the prep waves' extra intervals past nch + 2 (see steady_intervals)
        for (int q = nch + 3; q < steady_intervals(nch); ++q) __syncthreads();
        if (s_fin) {
#pragma unroll
            for (int jb = 0; jb < KB; ++jb)
                *reinterpret_cast<float4 *>(s_fin + srow + 16 * jb + 4 * g) =
                    make_float4(Z[jb][0], Z[jb][1], Z[jb][2], Z[jb][3]);
        }
        if (SUMMARY) {
            float *p_fin = cp.ws_p + sidx * NN;
#pragma unroll
            for (int jb = 0; jb < KB; ++jb)
                *reinterpret_cast<float4 *>(p_fin + srow + 16 * jb + 4 * g) =
                    make_float4(Zp[jb][0], Zp[jb][1], Zp[jb][2], Zp[jb][3]);
        }
    } else if (matrix_wave) {
        // ---------------- matrix wave: the triangular inverse of chunk q-1 ----------------
        // The same intervals and barriers as the prep waves (below): interval -1,
        // the S intervals of their loop and the ones left up to nch + 2.  It is
        // each interval's longest dependent path, so it takes the highest priority.
        __builtin_amdgcn_s_setprio(3);
        __syncthreads();  // interval -1: decay totals of chunk 0
        const int S = steady_intervals(nch);
        for (int q = 0; q < S; ++q) {
            K.template matrices<!SUMMARY, kMatWave>(sm.ops[(q + 2) % 3]);  // chunk q-1 (q >= 1)
            __syncthreads();
        }
        for (int q = S; q < nch + 3; ++q) {
            if (q == nch) K.template matrices<!SUMMARY, kMatWave>(sm.ops[(nch - 1) % 3]);
            __syncthreads();
        }
    } else {
        // ---------------- prep waves: loads, operands, chunk matrices ----------------
        // the zero half of (M_kk | 0) in every buffer, once (read after the
        // barriers that precede the first chain step)
        for (int i = (int)threadIdx.x - 64 * G::CW; i < 3 * 16 * 4; i += 64 * G::PW)
            *reinterpret_cast<uint2 *>(sm.ops[i >> 6].mkz + ((i >> 2) & 15) * kPRow +
                                       8 * (i & 3) + 4) = make_uint2(0u, 0u);
        // The prep waves bound each interval (the chain waves wait at the barrier),
        // so they win the issue arbitration on their SIMD.  Two workgroups on one
        // CU: at equal priority the older one wins every tie, finishes ~15% ahead
        // and leaves the other to run its tail alone; the workgroup in an odd slot
        // of its CU (HW_ID bits 19:16, the second one placed) takes one level more,
        // which evens out their finishing times.  Alone on a CU it changes nothing
        // (the order within the workgroup stays the same).
        if (!MW && workgroup_slot_odd()) __builtin_amdgcn_s_setprio(3);
        else __builtin_amdgcn_s_setprio(2);
        ProParams pro{};
        const int kch = h * NH + 64 * K.kh + 4 * lo;  // the lane's four keys
        if (FUSED) {
            const float4 q = *reinterpret_cast<const float4 *>(p.k_k + kch);
            pro.kk[0] = q.x; pro.kk[1] = q.y; pro.kk[2] = q.z; pro.kk[3] = q.w;
            const float4 s = *reinterpret_cast<const float4 *>(p.k_a + kch);
            pro.ka[0] = s.x; pro.ka[1] = s.y; pro.ka[2] = s.z; pro.ka[3] = s.w;
        }
        float rk[4] = {0.f, 0.f, 0.f, 0.f};
        if (EPI && !SUMMARY) {
            const float4 q = *reinterpret_cast<const float4 *>(p.epi.r_k + kch);
            rk[0] = q.x; rk[1] = q.y; rk[2] = q.z; rk[3] = q.w;
        }
        // (the parameters above are in registers before the ring's loads start,
        // so no wait for them is left inside the loop)
        __builtin_amdgcn_s_waitcnt(kWaitAllLoads);
        // Raw inputs of the next kPrefetch chunks stay in flight in a register ring.
        // Interval q (one barrier each) forms chunk q-1's matrices and prepares
        // chunk q from ring slot q % kPrefetch, which then receives chunk
        // q + kPrefetch; at its end, once slot q+1 has arrived, each wave scans
        // the decay of chunk q+1 over its four tokens and leaves its total in LDS
        // for the later waves (read after the barrier).  The intervals run in a
        // loop without branches inside its body, unrolled over whole turns of the
        // ring and entered with the ring in its steady state: every join or extra
        // back edge there makes the compiler's wait counts for the ring
        // conservative (it then waits for loads issued one interval earlier
        // instead of kPrefetch - 1).  So the loop runs whole trips,
        // S = steady_intervals(nch) >= nch intervals:
        //   - interval 0 forms the matrices of buffer 2, which nobody reads
        //     before prep fills it in interval 2 and matrices in interval 3;
        //   - intervals past nch - 1 prepare chunks made only of padding tokens
        //     (clamped loads).
        // Both are harmless because interval q writes only the buffers of
        // chunks q and q-1 while the chain waves read chunk q-2's.
        constexpr int kMat = MW ? kMatSplit : kMatInPrep;
        Raw<W32> xs[kPrefetch];
#pragma unroll
        for (int d = 0; d < kPrefetch; ++d) K.load(d, xs[d]);
        constexpr int kLoads = FUSED ? 5 : 6;  // loads per chunk (no kappa when fused)
        // the next interval consumes the oldest ring slot: let only the
        // (kPrefetch-1) younger chunks' loads stay in flight (stated explicitly,
        // since the compiler's count does not survive the loop's back edge)
        __builtin_amdgcn_s_waitcnt(wait_older_chunks(kLoads));
        float lp[4], lx[4];
        {
            float w[4];
            K.unpack_w(xs[0], K.ptok() < K.Tl, w);
            // this wave's slots that no earlier wave writes hold 1 for good
            if (g == 0) {
#pragma unroll
                for (int b = 0; b < 3; ++b)
                    if (b >= blk) sm.carry[K.kh][0][blk][b][lo] =
                        sm.carry[K.kh][1][blk][b][lo] = make_float4(1.f, 1.f, 1.f, 1.f);
            }
            K.scan(w, lp, lx, sm.carry[K.kh][0]);
        }
        __syncthreads();  // interval -1: decay totals of chunk 0
        static_assert(kUnroll % kPrefetch == 0, "the loop advances whole ring turns");
        const int S = steady_intervals(nch);
        for (int q0 = 0; q0 < S; q0 += kUnroll) {
#pragma unroll
            for (int d = 0; d < kUnroll; ++d) {
                const int q = q0 + d;
                Raw<W32> &x = xs[d % kPrefetch];
                // chunk q-1's matrices (q >= 1), then widen the slot, form chunk
                // q's operands and refill the slot with chunk q + kPrefetch
                // (clamped: always the same loads per interval; refilling before
                // the operands are formed keeps both live and costs the register
                // budget that lets two workgroups share a CU)
                K.template matrices<!SUMMARY, kMat>(sm.ops[(q + 2) % 3]);  // chunk q-1 (q >= 1)
                const auto u = K.unpack(x, q * kC + K.ptok() < K.Tl, pro);
                K.template prep<!SUMMARY>(u, sm.ops[q % 3], rk, lp, lx,
                                          sm.carry[K.kh][q & 1][blk]);
                K.load(q + kPrefetch, x);
                __builtin_amdgcn_s_waitcnt(wait_older_chunks(kLoads));
                float w[4];
                K.unpack_w(xs[(d + 1) % kPrefetch], (q + 1) * kC + K.ptok() < K.Tl, w);
                K.scan(w, lp, lx, sm.carry[K.kh][(q + 1) & 1]);
                __syncthreads();
            }
        }
        // the intervals left up to nch + 2: the last chunk's matrices if the loop
        // stopped at interval nch, then barriers only
        for (int q = S; q < nch + 3; ++q) {
            if (q == nch) K.template matrices<!SUMMARY, kMat>(sm.ops[(nch - 1) % 3]);
            __syncthreads();
        }
    }
}

// Entry states of the segments of one (b, h): S_in[0] = s0 (or 0) and
// S_in[g+1] = S_in[g] P_g + dS_g, in fp32.  The value rows i are independent,
// so each workgroup owns kCombineRows = 16 rows of one (b, h), and wave w forms
// columns 16w .. 16w+15 of them as one 16 x 16 tile of fp32 matrix-core
// products (v_mfma_f32_16x16x4_f32: the state rows as A, P_g's columns as B,
// the tile in the accumulator, dS_g its initial value), four partial chains
// of four products each.  Each product is small, so the chain of G - 1 of
// them is latency-bound:
//  - P_g and the tile's rows of dS_g are loaded three segments ahead into a
//    four-slot register ring; the loop is unrolled by four so that every slot
//    keeps its registers and the compiler's wait counts leave the younger
//    slots in flight;
//  - the slots are native vectors and both helpers are forced inline (else
//    the slots live in scratch memory);
//  - indices past the last transition are clamped, so every load is issued on
//    every path;
//  - P_g and the current state rows reach every wave through double buffers in
//    LDS, one barrier per segment.
// The products take k in the order k = 4kb + g (lane group g supplies the g-th
// k of product kb), so that a lane's B operands, P[4kb + g][16w + lo], sit in
// LDS rows 80 floats apart (conflict-free across the wave), and the state rows
// are kept with column 4kb + g at position 16g + kb, so a lane's sixteen A
// operands are four 16-byte reads.
constexpr int kCombineRows = 16;
constexpr int kCombineParts = kN / kCombineRows;
constexpr int kCombPStride = 80;  // floats per P row in LDS
constexpr int kCombSStride = 68;  // floats per state row in LDS

struct CombineSlot {
    f32x4 p0, p1, p2, p3;  // thread t's part of P_g: elements 4 (t + 256 m) .. +3, m = 0..3
    f32x4 d;               // dS_g at rows 4g + e of the block, column 16w + lo
};

__global__ __launch_bounds__(256) void segment_combine_kernel(ChunkedParams cp) {
    __shared__ __align__(16) float Pl[2][kN * kCombPStride];
    __shared__ __align__(16) float Sl[2][kCombineRows * kCombSStride];
    const long bh = blockIdx.x / kCombineParts;
    const int part = blockIdx.x - (int)bh * kCombineParts;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, lo = lane & 15;
    const int col = 16 * w + lo;                                      // this lane's column
    const long cell = (long)(kCombineRows * part + 4 * g) * kN + col;  // element 0's cell; e: + e kN
    const long slot0 = bh * cp.nseg * kN * kN;                        // segment 0 of (b, h)
    const int last = cp.nseg - 1;  // transitions and offsets exist for segments 0 .. last - 1
    // S_in of the current segment: element e = row 4g + e of the block, column col
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
    if (cp.p.s0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) st[e] = cp.p.s0[bh * kN * kN + cell + e * kN];
    }
    // where thread t puts its 4 float4 of P in LDS, and where a lane writes its
    // tile element e in the state rows (column col at position 16 (col & 3) + col / 4)
    int poff[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int i = 4 * (t + 256 * m);
        poff[m] = (i / kN) * kCombPStride + i % kN;
    }
    const int spos = 16 * (col & 3) + (col >> 2);
    auto issue = [&](CombineSlot &s, int sg) __attribute__((always_inline)) {
        const long o = slot0 + (long)min(sg, last - 1) * kN * kN;
        const f32x4 *pp = reinterpret_cast<const f32x4 *>(cp.ws_p + o) + t;
        s.p0 = pp[0];
        s.p1 = pp[256];
        s.p2 = pp[512];
        s.p3 = pp[768];
#pragma unroll
        for (int e = 0; e < 4; ++e) s.d[e] = cp.ws_ds[o + cell + e * kN];
        // keep the slots in issue order (the scheduler would otherwise move the
        // prologue's first slot behind the others and every wait would cover it)
        __builtin_amdgcn_sched_barrier(0);
    };
    // segment sg: store its entry state, issue the loads of segment sg + 3 into
    // nxt and, unless sg is the last, form the next entry state from cur.  Past
    // the last segment a step repeats the last store with the same values, so
    // every step issues the same memory operations and the loop needs no exit
    // in its body (exits there made the compiler wait for the whole ring).
    auto step = [&](CombineSlot &cur, CombineSlot &nxt, int sg) __attribute__((always_inline)) {
        const long o = slot0 + (long)min(sg, last) * kN * kN;
#pragma unroll
        for (int e = 0; e < 4; ++e) cp.ws_sin[o + cell + e * kN] = st[e];
        issue(nxt, sg + 3);
        const int buf = sg & 1;
        if (sg < last) {
            float *pl = Pl[buf];
            *reinterpret_cast<f32x4 *>(pl + poff[0]) = cur.p0;
            *reinterpret_cast<f32x4 *>(pl + poff[1]) = cur.p1;
            *reinterpret_cast<f32x4 *>(pl + poff[2]) = cur.p2;
            *reinterpret_cast<f32x4 *>(pl + poff[3]) = cur.p3;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sl[buf][(4 * g + e) * kCombSStride + spos] = st[e];
        }
        __syncthreads();
        if (sg < last) {
            // A operands: row lo of the block at columns 4kb + g, kb = 0..15
            const f32x4 *srow = reinterpret_cast<const f32x4 *>(&Sl[buf][lo * kCombSStride + 16 * g]);
            const f32x4 a4[4] = {srow[0], srow[1], srow[2], srow[3]};
            const float *pcol = &Pl[buf][g * kCombPStride + col];  // P[4kb + g][col]: + 4kb rows
            Acc4 acc[4] = {Acc4{cur.d}, Acc4::zero(), Acc4::zero(), Acc4::zero()};
#pragma unroll
            for (int kb = 0; kb < 16; ++kb)
                acc[kb & 3] = mfma_f32(a4[kb >> 2][kb & 3], pcol[4 * kb * kCombPStride], acc[kb & 3]);
            st = (acc[0].v + acc[1].v) + (acc[2].v + acc[3].v);
        }
    };
    CombineSlot s0, s1, s2, s3;
    issue(s0, 0);
    issue(s1, 1);
    issue(s2, 2);
    for (int sg = 0; sg <= last; sg += 4) {
        step(s0, s3, sg);
        step(s1, s0, sg + 1);
        step(s2, s1, sg + 2);
        step(s3, s2, sg + 3);
    }
}

}  // namespace

namespace {

int device_cu_count() {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Segments per sequence: split the time axis only when the (b, h) pairs alone
// leave at least half the compute units idle and each segment keeps at least
// 8 chunks (the split costs a summary pass over all but the last segment, and
// each pass fills and drains its pipeline).  G segments per (b, h) with
// B*H*G <= 2 CUs: two workgroups per compute unit, as LDS and registers allow
// (a pair shortens every segment's serial walk more than it slows each
// interval: B1 T65536 H40 1.73 -> 1.53 ms against one per CU, B4 T1024 H12
// 85 -> 67 us against no split; with the matrix-core combine, 8-chunk
// segments took B4 T1024 H12 from 51.2 to 49.3 us against 16-chunk ones).
void segment_plan(int B, int T, int H, int &nseg, int &seg_len) {
    nseg = 1;
    seg_len = T;
    const long bh = (long)B * H;
    const int cu = device_cu_count();
    if (T < 512 || 2 * bh > cu) return;
    int G = (int)(2 * cu / bh);
    G = min(G, T / 128);
    G = min(G, 64);
    if (G < 2) return;
    int L = (T + G - 1) / G;
    L = (L + kC - 1) / kC * kC;
    nseg = (T + L - 1) / L;
    seg_len = L;
    if (nseg < 2) {
        nseg = 1;
        seg_len = T;
    }
}

}  // namespace

size_t chunked_workspace_bytes(int B, int T, int H) {
    int nseg, seg_len;
    segment_plan(B, T, H, nseg, seg_len);
    if (nseg == 1) return 0;
    return (size_t)3 * B * H * nseg * kN * kN * sizeof(float);
}

// One launch of the head-size-64 kernel over `wgs` workgroups.  When every
// workgroup has a compute unit to itself, the variant with a matrix wave runs:
// alone on a CU an interval waits for the wave that forms the triangular
// inverse, and without its share of the operands that wave finishes sooner.
// With two workgroups per CU the eight-wave form keeps its register budget
// (a ninth wave would not leave room for the second workgroup).
template <bool EPI, bool SUMMARY, bool W32, bool FUSED, bool YADD>
hipError_t launch_chunked64(const ChunkedParams &cp, long wgs, hipStream_t stream) {
    if (wgs <= device_cu_count())
        hipLaunchKernelGGL((chunked_kernel<EPI, SUMMARY, W32, FUSED, YADD, 64, true>),
                           dim3((unsigned)wgs), dim3(kThreadsMW), 0, stream, cp);
    else
        hipLaunchKernelGGL((chunked_kernel<EPI, SUMMARY, W32, FUSED, YADD, 64, false>),
                           dim3((unsigned)wgs), dim3(kThreads), 0, stream, cp);
    return hipGetLastError();
}

template <bool W32, bool FUSED, bool YADD>
hipError_t launch_chunked_w(ChunkedParams cp, hipStream_t stream) {
    const ForwardArgs &p = cp.p;
    const long bh = (long)p.B * p.H;
    if (cp.nseg > 1) {
        const size_t slab = (size_t)bh * cp.nseg * kN * kN;
        cp.ws_p = static_cast<float *>(p.workspace);
        cp.ws_ds = cp.ws_p + slab;
        cp.ws_sin = cp.ws_ds + slab;
        // 1. transitions and offsets of every segment but the last
        cp.nseg_launch = cp.nseg - 1;
        hipError_t e =
            launch_chunked64<false, true, W32, FUSED, false>(cp, bh * cp.nseg_launch, stream);
        if (e != hipSuccess) return e;
        // 2. entry state of every segment
        hipLaunchKernelGGL(segment_combine_kernel, dim3((unsigned)(bh * kCombineParts)), dim3(256),
                           0, stream, cp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // 3. readouts and final states, all segments in parallel
    cp.nseg_launch = cp.nseg;
    if (p.epilogue) return launch_chunked64<true, false, W32, FUSED, YADD>(cp, bh * cp.nseg, stream);
    return launch_chunked64<false, false, W32, FUSED, YADD>(cp, bh * cp.nseg, stream);
}

// Head size 128: one workgroup per (b, h), no segments.
template <bool W32>
hipError_t launch_chunked128(ChunkedParams cp, hipStream_t stream) {
    const ForwardArgs &p = cp.p;
    cp.nseg = cp.nseg_launch = 1;
    cp.seg_len = p.T;
    const dim3 grid((unsigned)((long)p.B * p.H)), block(Geo<128>::threads);
    if (p.epilogue)
        hipLaunchKernelGGL((chunked_kernel<true, false, W32, false, false, 128, false>), grid, block, 0,
                           stream, cp);
    else
        hipLaunchKernelGGL((chunked_kernel<false, false, W32, false, false, 128, false>), grid, block, 0,
                           stream, cp);
    return hipGetLastError();
}

hipError_t launch_chunked(const ForwardArgs &p, hipStream_t stream) {
    ChunkedParams cp{};
    cp.p = p;
    // head size 128: plain forward only (the API routes the other entry points to
    // the scan), no stored states
    if (p.N == 128)
        return p.w32 ? launch_chunked128<true>(cp, stream) : launch_chunked128<false>(cp, stream);
    segment_plan(p.B, p.T, p.H, cp.nseg, cp.seg_len);
    // the fused prologue comes with bf16 decays only (the API refuses it with float32 w)
    if (p.fused) return launch_chunked_w<false, true, false>(cp, stream);
    if (p.y_add)
        return p.w32 ? launch_chunked_w<true, false, true>(cp, stream)
                     : launch_chunked_w<false, false, true>(cp, stream);
    return p.w32 ? launch_chunked_w<true, false, false>(cp, stream)
                 : launch_chunked_w<false, false, false>(cp, stream);
}

}  // namespace wkv7
