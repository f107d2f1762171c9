// Host side of librwkv7_wkv.so: argument validation and dispatch for the C ABI
// declared in include/rwkv7_wkv.h.  Every check runs before anything is
// enqueued, so a failed call launches nothing and writes nothing.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "wkv7_internal.h"

namespace wkv7 {
namespace {

// grid-stride, so that any state size fits a grid of at most 2^16 workgroups
__global__ void state_copy_kernel(const float4 *src, float4 *dst, size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        dst[i] = src ? src[i] : make_float4(0.f, 0.f, 0.f, 0.f);
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a * b * ... with overflow detection against SIZE_MAX / 2
bool mul_ok(size_t &acc, size_t x) {
    if (x != 0 && acc > (SIZE_MAX / 2) / x) return false;
    acc *= x;
    return true;
}

rwkv7_status check_epilogue(const rwkv7_epilogue *epi) {
    if (!epi) return RWKV7_OK;
    if (!epi->r_k) return RWKV7_ERR_NULL;
    if (!aligned16(epi->r_k) || (epi->ln_w && !aligned16(epi->ln_w)) ||
        (epi->ln_b && !aligned16(epi->ln_b)))
        return RWKV7_ERR_ALIGN;
    return RWKV7_OK;
}

EpilogueArgs to_epi(const rwkv7_epilogue *epi) {
    EpilogueArgs e{};
    if (epi) {
        e.ln_w = epi->ln_w;
        e.ln_b = epi->ln_b;
        e.r_k = epi->r_k;
        e.eps = epi->eps;
    }
    return e;
}

}  // namespace

hipError_t launch_state_copy(const float *s0, float *s_out, size_t count, hipStream_t stream) {
    const size_t n4 = count / 4;
    const size_t need = (n4 + 255) / 256;
    const unsigned blocks = (unsigned)(need < 65536 ? need : 65536);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(state_copy_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4 *>(s0), reinterpret_cast<float4 *>(s_out),
                       n4);
    return hipGetLastError();
}

}  // namespace wkv7

using namespace wkv7;

extern "C" {

int rwkv7_abi_version(void) { return RWKV7_ABI_VERSION; }

const char *rwkv7_status_str(rwkv7_status s) {
    switch (s) {
        case RWKV7_OK: return "ok";
        case RWKV7_ERR_NULL: return "a required pointer is NULL";
        case RWKV7_ERR_SHAPE: return "invalid shape (B, H >= 1, T >= 0, sizes must fit)";
        case RWKV7_ERR_DTYPE: return "unknown dtype or algorithm";
        case RWKV7_ERR_UNSUPPORTED:
            return "unsupported (head size, or algorithm/entry point for this dtype)";
        case RWKV7_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case RWKV7_ERR_ALIAS: return "an output overlaps an input";
        case RWKV7_ERR_WORKSPACE: return "workspace missing or too small";
        case RWKV7_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

// The kernels index a head's channels (h * N + i, the per-channel epilogue and
// prologue parameters) in 32 bits: H * N must stay below 2^31.
static bool heads_fit(int H, int N) { return (long long)H * N <= 0x7fffffffLL; }

static bool valid_dtype(rwkv7_dtype dt) {
    return dt == RWKV7_DT_F32 || dt == RWKV7_DT_BF16 || dt == RWKV7_DT_BF16_W32;
}

// AUTO: the chunked kernel for bf16 inputs at head size 64 (and at 128 where the
// entry point has a chunked kernel of that size: chunked128), else the scan.
static rwkv7_algo resolve_algo(rwkv7_algo algo, rwkv7_dtype dt, int N = kN,
                               bool chunked128 = false) {
    if (algo == RWKV7_ALGO_AUTO)
        return (dt != RWKV7_DT_F32 && (N == kN || (N == 128 && chunked128)) && kChunkedAvailable)
                   ? RWKV7_ALGO_CHUNKED
                   : RWKV7_ALGO_SCAN;
    return algo;
}

size_t rwkv7_wkv_forward_workspace(int B, int T, int H, int N, rwkv7_dtype dt, rwkv7_algo algo) {
    if (B < 1 || H < 1 || T < 0 || (N != 64 && N != 128)) return 0;
    if (!valid_dtype(dt)) return 0;
    if (resolve_algo(algo, dt, N) != RWKV7_ALGO_CHUNKED || T == 0 || N != kN) return 0;
    return chunked_workspace_bytes(B, T, H);
}

size_t rwkv7_wkv_forward_bidir_workspace(int B, int T, int H, int N, rwkv7_dtype dt,
                                         rwkv7_algo algo) {
    if (B < 1 || H < 1 || T <= 0 || (N != 64 && N != 128) || !valid_dtype(dt)) return 0;
    size_t n = 1;
    if (!mul_ok(n, (size_t)B) || !mul_ok(n, (size_t)T) || !mul_ok(n, (size_t)H) ||
        !mul_ok(n, (size_t)N * 4))
        return 0;
    return n + rwkv7_wkv_forward_workspace(B, T, H, N, dt, algo);
}

}  // extern "C"

// Bytes of the float32 readouts of a bidirectional call's reverse pass.
static size_t bidir_yrev_bytes(int B, int T, int H, int N) { return (size_t)B * T * H * N * 4; }

// rwkv7_wkv_forward; with s_ckpt (training forward, no epilogue) the states
// before every kCkpt-th token as well; with bidir the bidirectional forward
// (s0 / s_out hold two states per head).
static rwkv7_status forward_impl(const void *r, const void *w, const void *k, const void *v,
                                 const void *kappa, const void *a, const float *s0, void *y,
                                 float *s_out, float *s_ckpt, bool want_ckpt, bool bidir, int B,
                                 int T, int H, int N, rwkv7_dtype dt, rwkv7_algo algo,
                                 const rwkv7_epilogue *epi, void *workspace,
                                 size_t workspace_bytes, void *stream,
                                 const rwkv7_prologue *pro = nullptr) {
    if (!valid_dtype(dt)) return RWKV7_ERR_DTYPE;
    if (pro && dt == RWKV7_DT_BF16_W32) return RWKV7_ERR_UNSUPPORTED;
    if (algo != RWKV7_ALGO_AUTO && algo != RWKV7_ALGO_SCAN && algo != RWKV7_ALGO_CHUNKED)
        return RWKV7_ERR_DTYPE;
    if (N != 64 && N != 128) return RWKV7_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || T < 0 || !heads_fit(H, N)) return RWKV7_ERR_SHAPE;
    // the chunked kernel at head size 128 runs the plain and the training forward
    const bool chunked128 = N == 128 && !pro && !bidir;
    const rwkv7_algo al = resolve_algo(algo, dt, N, chunked128);
    if (al == RWKV7_ALGO_CHUNKED &&
        (dt == RWKV7_DT_F32 || (N != kN && !chunked128) || !kChunkedAvailable))
        return RWKV7_ERR_UNSUPPORTED;

    const size_t esz = dt == RWKV7_DT_F32 ? 4 : 2;
    size_t tok = 1, st = 1;
    if (!mul_ok(tok, (size_t)B) || !mul_ok(tok, (size_t)T) || !mul_ok(tok, (size_t)H) ||
        !mul_ok(tok, (size_t)N) || !mul_ok(tok, 4))
        return RWKV7_ERR_SHAPE;
    const size_t tok_w = dt == RWKV7_DT_BF16 ? tok / 2 : tok;  // bytes of w
    tok = tok / 4 * esz;                                       // bytes of the other vectors
    if (!mul_ok(st, (size_t)B) || !mul_ok(st, (size_t)H) || !mul_ok(st, (size_t)N * N * 4))
        return RWKV7_ERR_SHAPE;
    if ((size_t)B * H > 0x7fffffffu) return RWKV7_ERR_SHAPE;
    // one workgroup per head (scan: 4N threads; chunked: 512, 1024 at N = 128):
    // the grid's extent in threads must fit in 32 bits (T == 0 runs only the state copy)
    const size_t head_threads =
        al == RWKV7_ALGO_CHUNKED ? (N == 128 ? 1024 : 512) : (size_t)4 * N;
    if (T > 0 && (size_t)B * H * head_threads > 0xffffffffu) return RWKV7_ERR_SHAPE;
    const size_t st1 = st;  // bytes of one state per head
    if (bidir && !mul_ok(st, 2)) return RWKV7_ERR_SHAPE;
    size_t ck = st1;  // bytes of the stored states
    if (want_ckpt && !mul_ok(ck, (size_t)((T + kCkpt - 1) / kCkpt))) return RWKV7_ERR_SHAPE;

    // the six vectors, and the output gate of the fused prologue (kappa is
    // formed in the kernel then: its pointer is not used)
    const void *ins[7] = {r, w, k, v, pro ? nullptr : kappa, a, pro ? pro->g : nullptr};
    auto in_rng = [&](int i) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(ins[i]);
        return lo ? Range{lo, lo + (i == 1 ? tok_w : tok)} : Range{0, 0};
    };
    if (pro) {
        if (!pro->k_k || !pro->k_a) return RWKV7_ERR_NULL;
        if (!aligned16(pro->k_k) || !aligned16(pro->k_a)) return RWKV7_ERR_ALIGN;
    }
    if (T > 0) {
        for (int i = 0; i < 6; ++i)
            if (!ins[i] && !(pro && i == 4)) return RWKV7_ERR_NULL;
        if (!y) return RWKV7_ERR_NULL;
        if (want_ckpt && !s_ckpt) return RWKV7_ERR_NULL;
    }
    if (!want_ckpt || T == 0) s_ckpt = nullptr;
    rwkv7_status es = check_epilogue(epi);
    if (es != RWKV7_OK) return es;
    for (const void *p : ins)
        if (p && !aligned16(p)) return RWKV7_ERR_ALIGN;
    if ((y && !aligned16(y)) || (s0 && !aligned16(s0)) || (s_out && !aligned16(s_out)) ||
        (s_ckpt && !aligned16(s_ckpt)))
        return RWKV7_ERR_ALIGN;

    // outputs may not overlap inputs (s_out == s0 exactly is the in-place case)
    auto rng = [](const void *p, size_t n) {
        return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n};
    };
    if (T > 0) {
        const Range ry = rng(y, tok);
        for (int i = 0; i < 7; ++i)
            if (overlap(ry, in_rng(i))) return RWKV7_ERR_ALIAS;
        if (s0 && overlap(ry, rng(s0, st))) return RWKV7_ERR_ALIAS;
        if (s_out && overlap(ry, rng(s_out, st))) return RWKV7_ERR_ALIAS;
        if (epi) {
            const size_t pn = (size_t)H * N * 4;
            if (overlap(ry, rng(epi->r_k, pn)) || (epi->ln_w && overlap(ry, rng(epi->ln_w, pn))) ||
                (epi->ln_b && overlap(ry, rng(epi->ln_b, pn))))
                return RWKV7_ERR_ALIAS;
        }
    }
    if (s_out) {
        const Range rs = rng(s_out, st);
        if (T > 0)
            for (int i = 0; i < 7; ++i)
                if (overlap(rs, in_rng(i))) return RWKV7_ERR_ALIAS;
        if (s0 && s0 != s_out && overlap(rs, rng(s0, st))) return RWKV7_ERR_ALIAS;
        if (epi) {
            const size_t pn = (size_t)H * N * 4;
            if (overlap(rs, rng(epi->r_k, pn)) || (epi->ln_w && overlap(rs, rng(epi->ln_w, pn))) ||
                (epi->ln_b && overlap(rs, rng(epi->ln_b, pn))))
                return RWKV7_ERR_ALIAS;
        }
    }
    if (s_ckpt) {
        const Range rc = rng(s_ckpt, ck);
        for (int i = 0; i < 7; ++i)
            if (overlap(rc, in_rng(i))) return RWKV7_ERR_ALIAS;
        if (overlap(rc, rng(y, tok)) || (s0 && overlap(rc, rng(s0, st))) ||
            (s_out && overlap(rc, rng(s_out, st))))
            return RWKV7_ERR_ALIAS;
    }
    const size_t need = bidir ? rwkv7_wkv_forward_bidir_workspace(B, T, H, N, dt, al)
                              : rwkv7_wkv_forward_workspace(B, T, H, N, dt, al);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return RWKV7_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RWKV7_ERR_ALIGN;
        const Range rw = rng(workspace, need);
        for (int i = 0; i < 7; ++i)
            if (overlap(rw, in_rng(i))) return RWKV7_ERR_ALIAS;
        if (overlap(rw, rng(y, tok)) || (s0 && overlap(rw, rng(s0, st))) ||
            (s_out && overlap(rw, rng(s_out, st))) || (s_ckpt && overlap(rw, rng(s_ckpt, ck))))
            return RWKV7_ERR_ALIAS;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (!s_out || s_out == s0) return RWKV7_OK;
        return launch_state_copy(s0, s_out, st / 4, hs) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
    }

    ForwardArgs p{};
    p.r = r; p.w = w; p.k = k; p.v = v; p.kappa = kappa; p.a = a;
    p.s0 = s0; p.y = y; p.s_out = s_out;
    p.B = B; p.T = T; p.H = H; p.N = N;
    p.bf16 = dt != RWKV7_DT_F32;
    p.w32 = dt == RWKV7_DT_BF16_W32;
    p.epilogue = epi != nullptr;
    p.epi = to_epi(epi);
    p.workspace = workspace;
    p.workspace_bytes = workspace_bytes;
    p.s_ckpt = s_ckpt;
    if (pro) {
        p.fused = true;
        p.kappa = nullptr;
        p.k_k = pro->k_k;
        p.k_a = pro->k_a;
        p.g = pro->g;
    }
    auto run = [&](const ForwardArgs &q) {
        return al == RWKV7_ALGO_CHUNKED ? launch_chunked(q, hs) : launch_scan(q, hs);
    };
    if (!bidir) return run(p) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;

    // bidirectional: the reverse pass (tokens T-1 .. 0, second state of each head)
    // leaves float32 readouts in the workspace; the forward pass adds them to its
    // own before the epilogue
    const size_t yrev = bidir_yrev_bytes(B, T, H, N);
    const size_t heads_elems = st1 / 4;
    float *ws_y = static_cast<float *>(workspace);
    ForwardArgs rev = p;
    rev.reverse = true;
    rev.epilogue = false;
    rev.y_f32 = ws_y;
    rev.s0 = s0 ? s0 + heads_elems : nullptr;
    rev.s_out = s_out ? s_out + heads_elems : nullptr;
    rev.workspace = static_cast<char *>(workspace) + yrev;
    rev.workspace_bytes = workspace_bytes - yrev;
    if (run(rev) != hipSuccess) return RWKV7_ERR_HIP;
    ForwardArgs fwd = p;
    fwd.y_add = ws_y;
    fwd.workspace = rev.workspace;
    fwd.workspace_bytes = rev.workspace_bytes;
    return run(fwd) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

extern "C" {

rwkv7_status rwkv7_wkv_forward(const void *r, const void *w, const void *k, const void *v,
                               const void *kappa, const void *a, const float *s0, void *y,
                               float *s_out, int B, int T, int H, int N, rwkv7_dtype dt,
                               rwkv7_algo algo, const rwkv7_epilogue *epi, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return forward_impl(r, w, k, v, kappa, a, s0, y, s_out, nullptr, false, false, B, T, H, N,
                        dt, algo, epi, workspace, workspace_bytes, stream);
}

rwkv7_status rwkv7_wkv_forward_fused(const void *r, const void *w, const void *k,
                                     const void *v, const void *a, const rwkv7_prologue *pro,
                                     const float *s0, void *y, float *s_out, int B, int T, int H,
                                     int N, rwkv7_dtype dt, rwkv7_algo algo,
                                     const rwkv7_epilogue *epi, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (!pro) return RWKV7_ERR_NULL;
    return forward_impl(r, w, k, v, nullptr, a, s0, y, s_out, nullptr, false, false, B, T, H, N,
                        dt, algo, epi, workspace, workspace_bytes, stream, pro);
}

rwkv7_status rwkv7_wkv_forward_bidir(const void *r, const void *w, const void *k,
                                     const void *v, const void *kappa, const void *a,
                                     const float *s0, void *y, float *s_out, int B, int T, int H,
                                     int N, rwkv7_dtype dt, rwkv7_algo algo,
                                     const rwkv7_epilogue *epi, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    return forward_impl(r, w, k, v, kappa, a, s0, y, s_out, nullptr, false, true, B, T, H, N,
                        dt, algo, epi, workspace, workspace_bytes, stream);
}

rwkv7_status rwkv7_wkv_forward_train(const void *r, const void *w, const void *k,
                                     const void *v, const void *kappa, const void *a,
                                     const float *s0, void *y, float *s_out, float *s_ckpt,
                                     int B, int T, int H, int N, rwkv7_dtype dt,
                                     rwkv7_algo algo, void *workspace, size_t workspace_bytes,
                                     void *stream) {
    return forward_impl(r, w, k, v, kappa, a, s0, y, s_out, s_ckpt, true, false, B, T, H, N, dt,
                        algo, nullptr, workspace, workspace_bytes, stream);
}

// AUTO: the chunked backward for bf16 (also with an fp32 decay) at head size 64,
// else the token-by-token one.
static rwkv7_algo resolve_bwd_algo(rwkv7_algo algo, rwkv7_dtype dt, int N) {
    if (algo == RWKV7_ALGO_AUTO)
        return dt != RWKV7_DT_F32 && N == kN ? RWKV7_ALGO_CHUNKED : RWKV7_ALGO_SCAN;
    return algo;
}

size_t rwkv7_wkv_backward_workspace(int B, int T, int H, int N, rwkv7_dtype dt,
                                    rwkv7_algo algo) {
    if (B < 1 || H < 1 || T <= 0 || (N != 64 && N != 128)) return 0;
    if (!valid_dtype(dt)) return 0;
    if (algo != RWKV7_ALGO_AUTO && algo != RWKV7_ALGO_SCAN && algo != RWKV7_ALGO_CHUNKED) return 0;
    size_t n = 1;
    if (!mul_ok(n, (size_t)B) || !mul_ok(n, (size_t)H) ||
        !mul_ok(n, (size_t)((T + kCkpt - 1) / kCkpt)) || !mul_ok(n, (size_t)N * N * 4))
        return 0;
    if ((size_t)B * H > 0x7fffffffu) return 0;
    if (resolve_bwd_algo(algo, dt, N) != RWKV7_ALGO_CHUNKED)
        return backward_scan_workspace_bytes(B, T, H, N);
    if (N != kN) return 0;
    return backward_chunked_workspace_bytes(B, T, H);
}

rwkv7_status rwkv7_wkv_backward(const void *r, const void *w, const void *k, const void *v,
                                const void *kappa, const void *a, const void *dy,
                                const float *s_ckpt, const float *ds_T, void *dr, void *dw,
                                void *dk, void *dv, void *dkappa, void *da, float *ds0, int B,
                                int T, int H, int N, rwkv7_dtype dt, rwkv7_algo algo,
                                void *workspace, size_t workspace_bytes, void *stream) {
    if (!valid_dtype(dt)) return RWKV7_ERR_DTYPE;
    if (algo != RWKV7_ALGO_AUTO && algo != RWKV7_ALGO_SCAN && algo != RWKV7_ALGO_CHUNKED)
        return RWKV7_ERR_DTYPE;
    if (N != 64 && N != 128) return RWKV7_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || T < 0 || !heads_fit(H, N)) return RWKV7_ERR_SHAPE;
    const rwkv7_algo use = resolve_bwd_algo(algo, dt, N);
    // chunked: bf16, or bf16 with an fp32 decay, at head size 64; the
    // token-by-token kernel: every dtype, head size 64 or 128
    if (use == RWKV7_ALGO_CHUNKED && (dt == RWKV7_DT_F32 || N != kN))
        return RWKV7_ERR_UNSUPPORTED;
    const size_t esz = dt == RWKV7_DT_F32 ? 4 : 2;
    size_t tok = 1, st = 1;
    if (!mul_ok(tok, (size_t)B) || !mul_ok(tok, (size_t)T) || !mul_ok(tok, (size_t)H) ||
        !mul_ok(tok, (size_t)N) || !mul_ok(tok, esz))
        return RWKV7_ERR_SHAPE;
    // w and dw: float32 with an fp32 decay
    const size_t tokw = dt == RWKV7_DT_BF16_W32 ? 2 * tok : tok;
    if (!mul_ok(st, (size_t)B) || !mul_ok(st, (size_t)H) || !mul_ok(st, (size_t)N * N * 4))
        return RWKV7_ERR_SHAPE;
    size_t ck = st;
    if (!mul_ok(ck, (size_t)((T + kCkpt - 1) / kCkpt))) return RWKV7_ERR_SHAPE;
    if ((size_t)B * H > 0x7fffffffu) return RWKV7_ERR_SHAPE;

    const void *ins[7] = {r, w, k, v, kappa, a, dy};
    void *outs[6] = {dr, dw, dk, dv, dkappa, da};
    if (T > 0) {
        for (const void *p : ins)
            if (!p) return RWKV7_ERR_NULL;
        for (const void *p : outs)
            if (!p) return RWKV7_ERR_NULL;
        if (!s_ckpt) return RWKV7_ERR_NULL;
    }
    for (const void *p : ins)
        if (p && !aligned16(p)) return RWKV7_ERR_ALIGN;
    for (const void *p : outs)
        if (p && !aligned16(p)) return RWKV7_ERR_ALIGN;
    if ((s_ckpt && !aligned16(s_ckpt)) || (ds_T && !aligned16(ds_T)) || (ds0 && !aligned16(ds0)))
        return RWKV7_ERR_ALIGN;
    const bool chunked = use == RWKV7_ALGO_CHUNKED && T > 0;
    // the token-by-token kernel at N = 128 keeps partial sums in the workspace
    const bool scan_ws = !chunked && N == 128 && T > 0;
    const size_t ws_need =
        chunked || scan_ws ? rwkv7_wkv_backward_workspace(B, T, H, N, dt, use) : 0;
    if ((chunked || scan_ws) && ws_need == 0) return RWKV7_ERR_SHAPE;
    if (chunked && !backward_chunked_grid_ok(B, T, H)) return RWKV7_ERR_SHAPE;
    // token by token: 256-thread workgroups, one per head at N = 64 and four at
    // 128; the grid's extent in threads must fit in 32 bits (T == 0: the state copy only)
    if (!chunked && T > 0 && (size_t)B * H * (N == 128 ? 1024 : 256) > 0xffffffffu)
        return RWKV7_ERR_SHAPE;
    if (chunked || scan_ws) {
        if (!workspace || workspace_bytes < ws_need) return RWKV7_ERR_WORKSPACE;
        if (!aligned16(workspace)) return RWKV7_ERR_ALIGN;
    }

    // outputs overlap neither each other nor an input (ds0 == ds_T is the in-place case)
    auto rng = [](const void *p, size_t n) {
        return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n};
    };
    auto vbytes = [&](int i) { return i == 1 ? tokw : tok; };  // index 1: w / dw
    if (T > 0) {
        for (int o = 0; o < 6; ++o) {
            const Range ro = rng(outs[o], vbytes(o));
            for (int i = 0; i < 7; ++i)
                if (overlap(ro, rng(ins[i], vbytes(i)))) return RWKV7_ERR_ALIAS;
            for (int o2 = o + 1; o2 < 6; ++o2)
                if (overlap(ro, rng(outs[o2], vbytes(o2)))) return RWKV7_ERR_ALIAS;
            if (overlap(ro, rng(s_ckpt, ck)) || (ds_T && overlap(ro, rng(ds_T, st))) ||
                (ds0 && overlap(ro, rng(ds0, st))))
                return RWKV7_ERR_ALIAS;
        }
    }
    if (ds0) {
        const Range rd = rng(ds0, st);
        if (T > 0) {
            for (int i = 0; i < 7; ++i)
                if (overlap(rd, rng(ins[i], vbytes(i)))) return RWKV7_ERR_ALIAS;
            if (overlap(rd, rng(s_ckpt, ck))) return RWKV7_ERR_ALIAS;
        }
        if (ds_T && ds_T != ds0 && overlap(rd, rng(ds_T, st))) return RWKV7_ERR_ALIAS;
    }
    if (ws_need > 0) {  // the workspace is written: it overlaps no argument
        const Range rw = rng(workspace, ws_need);
        for (int i = 0; i < 7; ++i)
            if (overlap(rw, rng(ins[i], vbytes(i)))) return RWKV7_ERR_ALIAS;
        for (int o = 0; o < 6; ++o)
            if (overlap(rw, rng(outs[o], vbytes(o)))) return RWKV7_ERR_ALIAS;
        if (overlap(rw, rng(s_ckpt, ck)) || (ds_T && overlap(rw, rng(ds_T, st))) ||
            (ds0 && overlap(rw, rng(ds0, st))))
            return RWKV7_ERR_ALIAS;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (T == 0) {
        if (!ds0 || ds0 == ds_T) return RWKV7_OK;
        return launch_state_copy(ds_T, ds0, st / 4, hs) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
    }
    BackwardArgs p{};
    p.r = r; p.w = w; p.k = k; p.v = v; p.kappa = kappa; p.a = a; p.dy = dy;
    p.s_ckpt = s_ckpt; p.ds_T = ds_T;
    p.dr = dr; p.dw = dw; p.dk = dk; p.dv = dv; p.dkappa = dkappa; p.da = da;
    p.ds0 = ds0;
    p.B = B; p.T = T; p.H = H; p.N = N;
    p.bf16 = dt != RWKV7_DT_F32;
    p.w32 = dt == RWKV7_DT_BF16_W32;
    if (scan_ws) p.scan_ws = static_cast<float *>(workspace);
    if (chunked) {
        p.ds_ws = static_cast<uint16_t *>(workspace);
        return launch_backward_chunked(p, hs) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
    }
    return launch_backward(p, hs) == hipSuccess ? RWKV7_OK : RWKV7_ERR_HIP;
}

}  // extern "C"

// rwkv7_wkv_decode; with pro, fed from raw keys through the time-mix prologue
// (kappa unused) and gated by pro->g.
static rwkv7_status decode_impl(const void *r, const void *w, const void *k, const void *v,
                                const void *kappa, const void *a, float *state, void *y, int B,
                                int H, int N, rwkv7_dtype dt, const rwkv7_epilogue *epi,
                                void *stream, const rwkv7_prologue *pro) {
    if (!valid_dtype(dt)) return RWKV7_ERR_DTYPE;
    if (pro && dt == RWKV7_DT_BF16_W32) return RWKV7_ERR_UNSUPPORTED;
    if (N != 64 && N != 128) return RWKV7_ERR_UNSUPPORTED;
    if (B < 1 || H < 1 || !heads_fit(H, N)) return RWKV7_ERR_SHAPE;
    const size_t esz = dt == RWKV7_DT_F32 ? 4 : 2;
    size_t tok = 1, st = 1;
    if (!mul_ok(tok, (size_t)B) || !mul_ok(tok, (size_t)H) || !mul_ok(tok, (size_t)N * 4))
        return RWKV7_ERR_SHAPE;
    const size_t tok_w = dt == RWKV7_DT_BF16 ? tok / 2 : tok;  // bytes of w
    tok = tok / 4 * esz;                                       // bytes of the other vectors
    if (!mul_ok(st, (size_t)B) || !mul_ok(st, (size_t)H) || !mul_ok(st, (size_t)N * N * 4))
        return RWKV7_ERR_SHAPE;
    // one workgroup per head, 256 threads (1024 at N = 128): the grid's extent in
    // threads must fit in 32 bits
    if ((size_t)B * H * (N == 128 ? 1024 : 256) > 0xffffffffu) return RWKV7_ERR_SHAPE;
    // the six vectors (kappa unused with the prologue) and the prologue's gate
    const void *ins[7] = {r, w, k, v, pro ? nullptr : kappa, a, pro ? pro->g : nullptr};
    auto in_rng = [&](int i) {
        const uintptr_t lo = reinterpret_cast<uintptr_t>(ins[i]);
        return lo ? Range{lo, lo + (i == 1 ? tok_w : tok)} : Range{0, 0};
    };
    for (int i = 0; i < 6; ++i)
        if (!ins[i] && !(pro && i == 4)) return RWKV7_ERR_NULL;
    if (!state || !y) return RWKV7_ERR_NULL;
    if (pro && (!pro->k_k || !pro->k_a)) return RWKV7_ERR_NULL;
    rwkv7_status es = check_epilogue(epi);
    if (es != RWKV7_OK) return es;
    for (const void *p : ins)
        if (p && !aligned16(p)) return RWKV7_ERR_ALIGN;
    if (!aligned16(state) || !aligned16(y)) return RWKV7_ERR_ALIGN;
    if (pro && (!aligned16(pro->k_k) || !aligned16(pro->k_a))) return RWKV7_ERR_ALIGN;
    auto rng = [](const void *p, size_t n) {
        return Range{reinterpret_cast<uintptr_t>(p), reinterpret_cast<uintptr_t>(p) + n};
    };
    const Range ry = rng(y, tok), rs = rng(state, st);
    if (overlap(ry, rs)) return RWKV7_ERR_ALIAS;
    for (int i = 0; i < 7; ++i)
        if (overlap(ry, in_rng(i)) || overlap(rs, in_rng(i))) return RWKV7_ERR_ALIAS;
    if (pro) {
        const size_t pn = (size_t)H * N * 4;
        if (overlap(ry, rng(pro->k_k, pn)) || overlap(rs, rng(pro->k_k, pn)) ||
            overlap(ry, rng(pro->k_a, pn)) || overlap(rs, rng(pro->k_a, pn)))
            return RWKV7_ERR_ALIAS;
    }
    if (epi) {
        const size_t pn = (size_t)H * N * 4;
        const void *ps[3] = {epi->r_k, epi->ln_w, epi->ln_b};
        for (const void *p : ps)
            if (p && (overlap(ry, rng(p, pn)) || overlap(rs, rng(p, pn)))) return RWKV7_ERR_ALIAS;
    }
    DecodeArgs p{};
    p.r = r; p.w = w; p.k = k; p.v = v; p.kappa = kappa; p.a = a;
    p.state = state; p.y = y; p.B = B; p.H = H; p.N = N;
    p.bf16 = dt != RWKV7_DT_F32;
    p.w32 = dt == RWKV7_DT_BF16_W32;
    p.epilogue = epi != nullptr;
    p.epi = to_epi(epi);
    if (pro) {
        p.fused = true;
        p.kappa = nullptr;
        p.k_k = pro->k_k;
        p.k_a = pro->k_a;
        p.g = pro->g;
    }
    return launch_decode(p, static_cast<hipStream_t>(stream)) == hipSuccess ? RWKV7_OK
                                                                             : RWKV7_ERR_HIP;
}

extern "C" {

rwkv7_status rwkv7_wkv_decode(const void *r, const void *w, const void *k, const void *v,
                              const void *kappa, const void *a, float *state, void *y, int B,
                              int H, int N, rwkv7_dtype dt, const rwkv7_epilogue *epi,
                              void *stream) {
    return decode_impl(r, w, k, v, kappa, a, state, y, B, H, N, dt, epi, stream, nullptr);
}

rwkv7_status rwkv7_wkv_decode_fused(const void *r, const void *w, const void *k, const void *v,
                                    const void *a, const rwkv7_prologue *pro, float *state,
                                    void *y, int B, int H, int N, rwkv7_dtype dt,
                                    const rwkv7_epilogue *epi, void *stream) {
    if (!pro) return RWKV7_ERR_NULL;
    return decode_impl(r, w, k, v, nullptr, a, state, y, B, H, N, dt, epi, stream, pro);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// rwkv7_wkv_forward_noalloc: rwkv7_wkv_forward for callers that cannot
// allocate.  The workspace of the chunked path (three float32 64 x 64 states
// per (batch, head, time segment), present only when a long sequence of few
// heads is split into parallel segments) lives in `scratch`, a fixed device
// array of this library; every call on a device shares that device's copy.
// The split keeps at most two segments per compute unit, so on a 256-CU device
// the workspace never exceeds 3 x 512 x 16 KiB = 24 MiB.  Nothing in it needs
// to start at zero: each call writes every slot it reads.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)24 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of the current device's `scratch`, looked up once per
// device (with that device current).  In host code the array's name is only a
// host-side stand-in; kernels receive this address.
rwkv7_status scratch_address(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RWKV7_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return RWKV7_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return RWKV7_OK;
}

}  // namespace

extern "C" rwkv7_status rwkv7_wkv_forward_noalloc(const void *r, const void *w, const void *k,
                                                  const void *v, const void *kappa,
                                                  const void *a, const float *s0, void *y,
                                                  float *s_out, int B, int T, int H, int N,
                                                  rwkv7_dtype dt, rwkv7_algo algo,
                                                  const rwkv7_epilogue *epi, void *stream) {
    const size_t need = rwkv7_wkv_forward_workspace(B, T, H, N, dt, algo);
    if (need > kScratchBytes) return RWKV7_ERR_WORKSPACE;
    void *ws = nullptr;
    if (need > 0) {
        const rwkv7_status st = scratch_address(&ws);
        if (st != RWKV7_OK) return st;
    }
    return rwkv7_wkv_forward(r, w, k, v, kappa, a, s0, y, s_out, B, T, H, N, dt, algo, epi, ws,
                             need, stream);
}
