/*
 * rwkv7_wkv.h -- C ABI of the MI355X (gfx950) WKV7 library, librwkv7_wkv.so.
 *
 * The WKV7 recurrence is the generalised delta-rule state update of RWKV-7
 * "Goose".  Per (batch b, head h), with an N x N float32 state S whose row
 * index i is the VALUE index and whose column index j is the KEY index, each
 * token t computes
 *
 *     u      = S kappa_t                                  (state before the step)
 *     S      = S diag(w_t) - u (kappa_t * a_t)^T + v_t k_t^T
 *     y_t    = S r_t                                      (state after the step)
 *
 * Sources: RWKV-7 "Goose" author response (paperhub), numpy time_mixing
 * listing (the update, the readout, the per-head GroupNorm and the bonus);
 * ARWKV verdict (pith.science, arXiv 2501.15570), key_machinery field (the same
 * update in row-vector form); RWKV-7 "Goose" summary (paperlayer, arXiv
 * 2503.14456v2), §4 Method (diagonal-plus-rank-one transition, parallel
 * chunked form), §8 Speed and Memory (head size 64, float32 states,
 * constant-memory single-token inference, chunked pre-fill).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library allocates no device memory, keeps no mutable global state and
 *    may be called from several host threads on different streams.
 *  - Per-token vectors r, w, k, v, kappa, a and the output y are dense,
 *    C-order [B, T, H, N] (forward) or [B, H, N] (decode) in the element type
 *    `dt`.  kappa is the removal key (the normalised key of the pages), k the
 *    replacement key that is written, a the in-context learning rate, w the
 *    decay, r the receptance.  The library applies no transform to any of them.
 *  - States are float32 [B, H, N, N], row-major: state[b][h][i][j], i = value
 *    index, j = key index.
 *  - N = 64 (the head size the pages' kernels are tuned for) everywhere; N = 128
 *    also for rwkv7_wkv_decode, for both algorithms of rwkv7_wkv_forward (and
 *    rwkv7_wkv_forward_noalloc) and of rwkv7_wkv_forward_train (RWKV7_ALGO_AUTO
 *    picks the chunked one for bf16), for the token-by-token algorithm of
 *    rwkv7_wkv_backward (which RWKV7_ALGO_AUTO picks at 128), and for the scan
 *    algorithm of the bidirectional and fused entry points (RWKV7_ALGO_AUTO
 *    picks the scan there).  The chunked algorithm of the bidirectional and
 *    fused entry points and of the backward returns RWKV7_ERR_UNSUPPORTED at
 *    128.  B, H >= 1; T >= 0; H * N < 2^31 (RWKV7_ERR_SHAPE otherwise).  All
 *    offsets into tensors are 64-bit.
 *  - Every pointer must be 16-byte aligned.
 *  - All validation runs on the host, synchronously, before anything is
 *    enqueued: on any error nothing is launched and nothing is written.
 *    Kernel faults surface at the caller's next synchronisation.  No C++
 *    exception crosses this interface.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    the call returns without waiting.
 *  - Numerics: float32 state and accumulation; y is rounded to nearest even
 *    when dt is bf16; kappa is used exactly as given (not renormalised); a is
 *    not clamped.
 *  - Non-finite inputs propagate, never across (batch, head) pairs: a NaN or
 *    Inf in token t's inputs of one pair reaches that pair's readouts from
 *    token t on (where the recurrence carries it) and its final state.  The
 *    scan and decode leave every earlier readout as it would be without it.
 *    RWKV7_ALGO_CHUNKED works on chunks of 16 tokens whose tokens meet in one
 *    matrix product (where 0 * NaN is NaN): the readouts of the tokens of t's
 *    chunk before t (tokens 16 floor(t/16) .. t-1) may become non-finite too;
 *    earlier chunks are unaffected.
 */
#ifndef RWKV7_WKV_H
#define RWKV7_WKV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RWKV7_ABI_VERSION 2

typedef enum {
    RWKV7_OK = 0,
    RWKV7_ERR_NULL = 1,        /* a required pointer is NULL                         */
    RWKV7_ERR_SHAPE = 2,       /* B < 1, H < 1, T < 0, or a size overflows            */
    RWKV7_ERR_DTYPE = 3,       /* unknown dtype / algo value                          */
    RWKV7_ERR_UNSUPPORTED = 4, /* head size, or algo/entry not available for dtype    */
    RWKV7_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                    */
    RWKV7_ERR_ALIAS = 6,       /* an output overlaps an input (other than s_out==s0) */
    RWKV7_ERR_WORKSPACE = 7,   /* workspace missing or smaller than required          */
    RWKV7_ERR_HIP = 8          /* the HIP runtime refused a launch                    */
} rwkv7_status;

typedef enum {
    RWKV7_DT_F32 = 0,      /* every per-token vector (and y) float32                   */
    RWKV7_DT_BF16 = 1,     /* every per-token vector (and y) bfloat16                  */
    RWKV7_DT_BF16_W32 = 2  /* bfloat16, except the decay w, which is float32: slow
                              forgetting (w near 1) survives the input rounding.  The
                              RWKV-7 "Goose" author response (paperhub) names precision
                              sensitivity of the kernel; with w in (0.99, 1), bf16 rounds
                              most decays to exactly 1.  Forward, training forward,
                              bidirectional forward, decode, and both backward
                              algorithms (whose dw is then float32 too); the fused
                              prologue returns RWKV7_ERR_UNSUPPORTED.                   */
} rwkv7_dtype;

typedef enum {
    RWKV7_ALGO_AUTO = 0,    /* CHUNKED for bf16, SCAN for f32                          */
    RWKV7_ALGO_SCAN = 1,    /* token-by-token recurrence, state kept on chip           */
    RWKV7_ALGO_CHUNKED = 2  /* chunked-parallel form on bf16 MFMA, float32 state;
                               bf16 only.  Domain of the decay: 2^-6 <= w <= 1.  Inside
                               a 16-token chunk the form divides by products of up to
                               16 decays (down to w^16 >= 2^-96, far inside the float32
                               and bf16 exponent range); below about w = 0.0043 they
                               underflow and the results are not finite.  The library
                               does not read the data, so it cannot reject such w; the
                               pages' parameterisation keeps w above 0.545.  The scan
                               and decode accept any w.                                  */
} rwkv7_algo;

/*
 * Optional fused epilogue: per-head GroupNorm of y over the N value channels
 * (mean and population variance, eps inside the square root, then the
 * per-channel affine ln_w, ln_b over the flattened H*N channels), followed by
 * the current-token bonus (sum_j r_j k_j r_k[h*N+j]) * v_i added after the
 * norm.  Source: RWKV-7 "Goose" author response (paperhub), numpy
 * time_mixing listing (group_norm with eps 64e-5 and the bonus line);
 * RWKV-7 "Goose" summary, App. F (per-head normalisation after receptance).
 * All three arrays are float32 device pointers of H*N entries.  ln_w == NULL
 * means all ones, ln_b == NULL all zeros; r_k is required.  The state is never
 * affected by the epilogue.
 */
typedef struct {
    const float *ln_w;
    const float *ln_b;
    const float *r_k;
    float eps; /* the pages use 64e-5 */
} rwkv7_epilogue;

/*
 * Forward over T tokens for B independent sequences (prefill).
 *   r, w, k, v, kappa, a : [B,T,H,N] in dt (inputs)
 *   s0    : [B,H,N,N] float32 initial state, or NULL for a zero state
 *   y     : [B,T,H,N] in dt (output; after the epilogue when epi != NULL)
 *   s_out : [B,H,N,N] float32 final state S_T, or NULL to skip it; may equal s0
 *           (updated in place); any other overlap with an input is an error
 *   epi   : NULL, or the fused epilogue above
 *   workspace / workspace_bytes : device scratch of at least
 *           rwkv7_wkv_forward_workspace(...) bytes (may be NULL when that is 0)
 * T == 0: y is untouched and s_out receives s0 (or zeros).
 */
rwkv7_status rwkv7_wkv_forward(const void *r, const void *w, const void *k, const void *v,
                               const void *kappa, const void *a, const float *s0, void *y,
                               float *s_out, int B, int T, int H, int N, rwkv7_dtype dt,
                               rwkv7_algo algo, const rwkv7_epilogue *epi, void *workspace,
                               size_t workspace_bytes, void *stream);

/* Bytes of device workspace rwkv7_wkv_forward needs for this problem (0 if none).
 * The chunked path splits long sequences of few heads into segments that run
 * in parallel (their transitions and offsets are combined exactly, by the
 * linearity of the state update in the entry state); the split, and so this
 * size, depends on the compute-unit count of the current device: query it with
 * the device current that the forward call will run on. */
size_t rwkv7_wkv_forward_workspace(int B, int T, int H, int N, rwkv7_dtype dt,
                                   rwkv7_algo algo);

/*
 * rwkv7_wkv_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same arguments without the workspace.  The workspace the chunked path
 * needs for long sequences of few heads comes from a fixed 24 MiB device array
 * of the library (one per device, held until the process ends); its address is
 * looked up once per device on the first call with that device current.  The
 * call itself allocates nothing.
 * Errors: those of rwkv7_wkv_forward, and RWKV7_ERR_WORKSPACE when
 * rwkv7_wkv_forward_workspace(...) for these arguments exceeds 24 MiB (it does
 * not on a device of up to 256 compute units).
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (several streams or host threads) race on it and must be
 * serialised by the caller; calls whose workspace size is 0 do not touch it.
 */
rwkv7_status rwkv7_wkv_forward_noalloc(const void *r, const void *w, const void *k,
                                       const void *v, const void *kappa, const void *a,
                                       const float *s0, void *y, float *s_out, int B, int T,
                                       int H, int N, rwkv7_dtype dt, rwkv7_algo algo,
                                       const rwkv7_epilogue *epi, void *stream);

/*
 * Fused time-mix prologue and output gate (RWKV-7 "Goose" author response,
 * paperhub, numpy time_mixing listing): from raw keys k the kernels form
 *   kappa = (k * k_k) / max(||k * k_k||, 1e-12)   (per head, over its N channels)
 *   k     <- k + k * (a - 1) * k_a                 (written and used by the bonus)
 * run the recurrence, apply the optional epilogue, then multiply y by g.
 *   k_k, k_a : [H*N] float32 per-channel parameters (required)
 *   g        : [B,T,H,N] in dt, or NULL for no gate
 */
typedef struct {
    const float *k_k;
    const float *k_a;
    const void *g;
} rwkv7_prologue;

/*
 * rwkv7_wkv_forward fed from raw keys: r, w, k (raw), v, a : [B,T,H,N] in dt
 * (float32 or bfloat16; RWKV7_DT_BF16_W32 returns RWKV7_ERR_UNSUPPORTED); no
 * kappa argument.  pro is required.  Workspace, s0, s_out, y, the epilogue and
 * the errors as rwkv7_wkv_forward (query the workspace there); g counts as an
 * input for the overlap checks.
 */
rwkv7_status rwkv7_wkv_forward_fused(const void *r, const void *w, const void *k,
                                     const void *v, const void *a, const rwkv7_prologue *pro,
                                     const float *s0, void *y, float *s_out, int B, int T, int H,
                                     int N, rwkv7_dtype dt, rwkv7_algo algo,
                                     const rwkv7_epilogue *epi, void *workspace,
                                     size_t workspace_bytes, void *stream);

/*
 * Bidirectional forward: the recurrence is run twice over the same inputs,
 * once over tokens 0 .. T-1 and once over tokens T-1 .. 0, and the two
 * readouts of each token are added; the optional epilogue then applies to the
 * sum.  Source: RWKV-7 "Goose" summary, §9 Multimodal Experiments (AudioRWKV-7
 * uses a bidirectional RWKV-7); the page gives no formula, and the plain
 * reading taken is this sum of a causal and an anti-causal pass.
 *   s0, s_out : [2,B,H,N,N] float32 (index 0: forward pass, 1: reverse pass),
 *               or NULL; s_out may equal s0 (in place).  The reverse pass's final
 *               state is the one after token 0.
 *   workspace  : at least rwkv7_wkv_forward_bidir_workspace(...) bytes (the
 *               reverse pass's float32 readouts, plus what the chunked path needs)
 * Everything else as rwkv7_wkv_forward.
 */
rwkv7_status rwkv7_wkv_forward_bidir(const void *r, const void *w, const void *k,
                                     const void *v, const void *kappa, const void *a,
                                     const float *s0, void *y, float *s_out, int B, int T, int H,
                                     int N, rwkv7_dtype dt, rwkv7_algo algo,
                                     const rwkv7_epilogue *epi, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Bytes of device workspace rwkv7_wkv_forward_bidir needs (0 for T == 0). */
size_t rwkv7_wkv_forward_bidir_workspace(int B, int T, int H, int N, rwkv7_dtype dt,
                                         rwkv7_algo algo);

/*
 * One token for each of B resident states (single-token inference, the
 * recurrence at T = 1 with the state read from and written back to HBM).
 * Head size N = 64 or 128 (RWKV-7 "Goose" summary, §8 Speed and Memory: the
 * pages' kernels are tuned for 64 and lose efficiency at larger heads).
 *   r, w, k, v, kappa, a : [B,H,N] in dt
 *   state : [B,H,N,N] float32, updated in place (for a layer-major pool the
 *           caller passes the layer's slice)
 *   y     : [B,H,N] in dt, must not overlap any other argument
 * Source: RWKV-7 "Goose" summary, §8 Speed and Memory (constant-memory
 * single-token inference); RWKV-X verdict (pith.science, arXiv 2504.21463):
 * RWKV-7 keeps no KV cache, only this state.
 */
rwkv7_status rwkv7_wkv_decode(const void *r, const void *w, const void *k, const void *v,
                              const void *kappa, const void *a, float *state, void *y, int B,
                              int H, int N, rwkv7_dtype dt, const rwkv7_epilogue *epi,
                              void *stream);

/* ---------------------------------------------------------------------------
 * Training path: forward with state storage, and the backward pass.
 * Source: RWKV-7 "Goose" summary, §8 Speed and Memory (forward inference with
 * state storage, then a backward computation); RWKV-7 "Goose" author response
 * (paperhub), answer on numerical precision (an fp32 gradient kernel and a
 * faster bf16 chunked one).  The pages give timings and error levels, not the
 * algorithm: the states stored here are the fp32 states at every 16th token,
 * and the backward recomputes the states in between from them.
 * ------------------------------------------------------------------------- */

/* Tokens between stored states. */
#define RWKV7_CKPT_INTERVAL 16

/*
 * rwkv7_wkv_forward without epilogue (the normalisation and bonus are separate
 * operations when training) that also stores
 *   s_ckpt : [B,H,C,N,N] float32, C = ceil(T / RWKV7_CKPT_INTERVAL):
 *            s_ckpt[b,h,c] = the state before token 16c (c = 0: s0, or zeros)
 * All other arguments, the workspace and the errors are those of
 * rwkv7_wkv_forward (query the workspace with rwkv7_wkv_forward_workspace).
 * s_ckpt must not overlap any other argument; it may be NULL only when T == 0.
 */
rwkv7_status rwkv7_wkv_forward_train(const void *r, const void *w, const void *k,
                                     const void *v, const void *kappa, const void *a,
                                     const float *s0, void *y, float *s_out, float *s_ckpt,
                                     int B, int T, int H, int N, rwkv7_dtype dt,
                                     rwkv7_algo algo, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * Gradients of L = sum_t <y_t, dy_t> + <S_T, ds_T> with respect to the inputs
 * of rwkv7_wkv_forward_train (without epilogue):
 *   r, w, k, v, kappa, a : [B,T,H,N] in dt, the forward's inputs (with
 *            RWKV7_DT_BF16_W32: w float32, the rest bfloat16)
 *   dy     : [B,T,H,N] in dt (bfloat16 for RWKV7_DT_BF16_W32), the cotangent of y
 *   s_ckpt : [B,H,C,N,N] float32 from rwkv7_wkv_forward_train on these inputs
 *   ds_T   : [B,H,N,N] float32 cotangent of the final state, or NULL (zero)
 *   dr, dw, dk, dv, dkappa, da : [B,T,H,N] in dt (outputs; for
 *            RWKV7_DT_BF16_W32 dw is float32 and the rest bfloat16)
 *   ds0    : [B,H,N,N] float32 gradient for s0 (output), or NULL to skip it;
 *            may equal ds_T (in place)
 *   algo   : RWKV7_ALGO_SCAN: token by token in fp32 VALU (states recomputed
 *              from s_ckpt), every dtype, head size 64 or 128.  At 128 each
 *              head's value rows are split over four workgroups whose partial
 *              sums over rows (of dr, dk, dw, dkappa, da) meet in the workspace
 *              and are added in a fixed order by a second kernel; the sequence
 *              is cut into slices of whole 16-token intervals whose partial
 *              sums stay within 256 MiB, walked last to first with the state
 *              cotangent carried between them;
 *            RWKV7_ALGO_CHUNKED: bf16 or bf16 with float32 w at head size 64
 *              (f32, or N = 128, refused with RWKV7_ERR_UNSUPPORTED); the
 *              chunked form on bf16 MFMA with fp32 accumulation: a reverse
 *              pass over the 16-token chunks carries the state cotangent and
 *              stores it at the end of every eighth chunk (the last of each
 *              group of 8) in the workspace, then the groups' gradients are
 *              formed in parallel, each group walked last to first from its
 *              stored cotangent and the stored states;
 *            RWKV7_ALGO_AUTO: CHUNKED for bf16 and bf16 with float32 w at head
 *              size 64, SCAN otherwise.
 *   workspace / workspace_bytes : device scratch of at least
 *            rwkv7_wkv_backward_workspace(...) bytes (CHUNKED: 8 KiB per head
 *            and group of 8 chunks, the decayed exit cotangent of the group's
 *            last chunk in bf16; SCAN: none
 *            at head size 64; at 128, 5 x 4 float32 per element of a slice,
 *            B*H*128*128*4 bytes more when there are several slices; may be
 *            NULL when that is 0); it must not overlap any other argument.
 * Gradients are rounded once to dt.  The six gradient outputs must not
 * overlap each other or any input.  T == 0: ds0 receives ds_T (or zeros).
 * The chunked form is the derivative of the chunked forward of the RWKV-7
 * "Goose" summary, §4 Method (parallel chunked form of the
 * diagonal-plus-rank-one transition); its algebra is stated with the kernels.
 */
rwkv7_status rwkv7_wkv_backward(const void *r, const void *w, const void *k, const void *v,
                                const void *kappa, const void *a, const void *dy,
                                const float *s_ckpt, const float *ds_T, void *dr, void *dw,
                                void *dk, void *dv, void *dkappa, void *da, float *ds0, int B,
                                int T, int H, int N, rwkv7_dtype dt, rwkv7_algo algo,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace rwkv7_wkv_backward needs (0 if none; 0 also for
 * invalid arguments). */
size_t rwkv7_wkv_backward_workspace(int B, int T, int H, int N, rwkv7_dtype dt,
                                    rwkv7_algo algo);

/*
 * rwkv7_wkv_decode fed from raw keys through the fused time-mix prologue
 * (rwkv7_prologue above; g is [B,H,N] in dt or NULL): r, w, k (raw), v, a :
 * [B,H,N] in dt (float32 or bfloat16); no kappa argument.  N = 64 or 128.
 * State, y, epilogue and errors as rwkv7_wkv_decode.
 */
rwkv7_status rwkv7_wkv_decode_fused(const void *r, const void *w, const void *k, const void *v,
                                    const void *a, const rwkv7_prologue *pro, float *state,
                                    void *y, int B, int H, int N, rwkv7_dtype dt,
                                    const rwkv7_epilogue *epi, void *stream);

/*
 * Measurement helper, not a step of the method: copies `bytes` bytes from src
 * to dst (device pointers, caller-owned) with whole 1 KiB wave accesses and
 * non-temporal loads and stores, every byte read and written once.  Its rate
 * is the HBM ceiling for a stream that reads and writes each byte once, which
 * is the traffic of the decode step.
 * bytes == 0 launches nothing.  Errors: RWKV7_ERR_NULL (a NULL pointer),
 * RWKV7_ERR_ALIGN (a pointer not 16-byte aligned), RWKV7_ERR_SHAPE (bytes not
 * a multiple of 16, or more than 2^31 workgroups of 8 KiB), RWKV7_ERR_ALIAS
 * (the ranges overlap), RWKV7_ERR_HIP (the launch failed).  Enqueued on
 * `stream` (NULL = default stream); returns before the copy completes.
 */
rwkv7_status rwkv7_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *rwkv7_status_str(rwkv7_status s);

/* RWKV7_ABI_VERSION of the built library. */
int rwkv7_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RWKV7_WKV_H */
