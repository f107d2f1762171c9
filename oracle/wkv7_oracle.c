/*
 * WKV7 oracle: a plain, slow CPU evaluation of the RWKV-7 state recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU path.
 *
 * What it computes, per (batch b, head h), for t = 0 .. T-1, with the state
 * S[i][j] (i = value index, j = key index), all arithmetic in the REAL type
 * (double for the oracle proper, float for the fp32 twin):
 *
 *   u[i]    = sum_j S[i][j] * kappa_t[j]                       (state before the step)
 *   S[i][j] = S[i][j]*w_t[j] - u[i]*(kappa_t[j]*a_t[j]) + v_t[i]*k_t[j]
 *   z[i]    = sum_j S[i][j] * r_t[j]                           (state after the step)
 *   optional epilogue (per-head GroupNorm, then the current-token bonus):
 *     mu = mean_i z[i];  var = mean_i (z[i]-mu)^2
 *     z[i] = (z[i]-mu)/sqrt(var+eps)*ln_w[h*N+i] + ln_b[h*N+i]
 *            + (sum_j r_t[j]*k_t[j]*r_k[h*N+j]) * v_t[i]
 *   y_t[i]  = z[i]
 *
 * Sources:
 *  - RWKV-7 "Goose" author response (paperhub), the numpy time_mixing
 *    listing: the state update (decay on the key columns, removal along the
 *    normalised key with rate a evaluated on the old state, write of v k^T),
 *    the receptance readout on the new state, the per-head GroupNorm with
 *    population variance and eps inside the square root, and the bonus term
 *    added after the normalisation.
 *  - ARWKV verdict (pith.science, arXiv 2501.15570), key_machinery field: the
 *    same update in row-vector form, S_t = S_{t-1}(diag(w) - kappa^T(a*kappa))
 *    + v^T k.
 *  - RWKV-7 "Goose" summary (paperlayer, arXiv 2503.14456v2), App. F: decay,
 *    removal, addition, then query with receptance.
 *
 * Layout: per-token vectors [B, T, H, N] C-order; states [B, H, N, N];
 * ln_w, ln_b, r_k each [H*N].  s0 == NULL means a zero initial state.
 * Threads (POSIX) split the independent (b, h) pairs.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    const void *r, *w, *k, *v, *kappa, *a, *s0;
    void *y, *s_out;
    long B, T, H, N;
    const void *ln_w, *ln_b, *r_k;
    double eps;
    int epilogue;
    long next;            /* next (b,h) index to process */
    int failed;
    pthread_mutex_t lock;
} oracle_job;

#define DEFINE_HEAD_RUNNER(NAME, REAL, SQRT)                                              \
static int NAME(oracle_job *J, long bh)                                                   \
{                                                                                         \
    const long B = J->B, T = J->T, H = J->H, N = J->N;                                    \
    const long b = bh / H, h = bh % H;                                                    \
    const REAL *r = (const REAL *)J->r, *w = (const REAL *)J->w, *k = (const REAL *)J->k; \
    const REAL *v = (const REAL *)J->v, *kap = (const REAL *)J->kappa;                    \
    const REAL *a = (const REAL *)J->a, *s0 = (const REAL *)J->s0;                        \
    REAL *y = (REAL *)J->y, *s_out = (REAL *)J->s_out;                                    \
    const REAL *ln_w = (const REAL *)J->ln_w, *ln_b = (const REAL *)J->ln_b;              \
    const REAL *r_k = (const REAL *)J->r_k;                                               \
    (void)B;                                                                              \
    REAL *S = (REAL *)malloc(sizeof(REAL) * N * N);                                       \
    REAL *u = (REAL *)malloc(sizeof(REAL) * N);                                           \
    REAL *z = (REAL *)malloc(sizeof(REAL) * N);                                           \
    if (!S || !u || !z) { free(S); free(u); free(z); return -1; }                         \
    const long sbase = (b * H + h) * N * N;                                               \
    if (s0) memcpy(S, s0 + sbase, sizeof(REAL) * N * N);                                  \
    else memset(S, 0, sizeof(REAL) * N * N);                                              \
    for (long t = 0; t < T; ++t) {                                                        \
        const long o = ((b * T + t) * H + h) * N;                                         \
        for (long i = 0; i < N; ++i) {                                                    \
            REAL acc = 0;                                                                 \
            for (long j = 0; j < N; ++j) acc += S[i * N + j] * kap[o + j];                \
            u[i] = acc;                                                                   \
        }                                                                                 \
        for (long i = 0; i < N; ++i)                                                      \
            for (long j = 0; j < N; ++j)                                                  \
                S[i * N + j] = S[i * N + j] * w[o + j] - u[i] * (kap[o + j] * a[o + j])   \
                               + v[o + i] * k[o + j];                                     \
        for (long i = 0; i < N; ++i) {                                                    \
            REAL acc = 0;                                                                 \
            for (long j = 0; j < N; ++j) acc += S[i * N + j] * r[o + j];                  \
            z[i] = acc;                                                                   \
        }                                                                                 \
        if (J->epilogue) {                                                                \
            REAL mu = 0, var = 0, bonus = 0;                                              \
            for (long i = 0; i < N; ++i) mu += z[i];                                      \
            mu /= (REAL)N;                                                                \
            for (long i = 0; i < N; ++i) var += (z[i] - mu) * (z[i] - mu);                \
            var /= (REAL)N;                                                               \
            const REAL inv = (REAL)1 / SQRT(var + (REAL)J->eps);                          \
            for (long j = 0; j < N; ++j) bonus += r[o + j] * k[o + j] * r_k[h * N + j];   \
            for (long i = 0; i < N; ++i) {                                                \
                REAL g = ln_w ? ln_w[h * N + i] : (REAL)1;                                \
                REAL c = ln_b ? ln_b[h * N + i] : (REAL)0;                                \
                z[i] = (z[i] - mu) * inv * g + c + bonus * v[o + i];                      \
            }                                                                             \
        }                                                                                 \
        for (long i = 0; i < N; ++i) y[o + i] = z[i];                                     \
    }                                                                                     \
    if (s_out) memcpy(s_out + sbase, S, sizeof(REAL) * N * N);                            \
    free(S); free(u); free(z);                                                            \
    return 0;                                                                             \
}

DEFINE_HEAD_RUNNER(run_head_f64, double, sqrt)
DEFINE_HEAD_RUNNER(run_head_f32, float, sqrtf)

typedef struct { oracle_job *job; int (*fn)(oracle_job *, long); } worker_arg;

static void *worker(void *p)
{
    worker_arg *wa = (worker_arg *)p;
    oracle_job *J = wa->job;
    const long total = J->B * J->H;
    for (;;) {
        long idx;
        pthread_mutex_lock(&J->lock);
        idx = J->next++;
        pthread_mutex_unlock(&J->lock);
        if (idx >= total) break;
        if (wa->fn(J, idx) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

static int run(oracle_job *J, int nthreads, int (*fn)(oracle_job *, long))
{
    if (J->B < 0 || J->T < 0 || J->H < 0 || J->N <= 0) return -2;
    if (J->epilogue && !J->r_k) return -3;
    const long total = J->B * J->H;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > total) nthreads = total > 0 ? (int)total : 1;
    J->next = 0;
    J->failed = 0;
    pthread_mutex_init(&J->lock, NULL);
    worker_arg wa = {J, fn};
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) return -1;
    int started = 0;
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[started], NULL, worker, &wa) == 0) ++started;
    worker(&wa);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J->lock);
    return J->failed ? -1 : 0;
}

#define DEFINE_ENTRY(NAME, REAL, FN)                                                      \
int NAME(const REAL *r, const REAL *w, const REAL *k, const REAL *v, const REAL *kappa,   \
         const REAL *a, const REAL *s0, REAL *y, REAL *s_out, long B, long T, long H,     \
         long N, const REAL *ln_w, const REAL *ln_b, const REAL *r_k, double eps,         \
         int epilogue, int nthreads)                                                      \
{                                                                                         \
    oracle_job J;                                                                         \
    memset(&J, 0, sizeof J);                                                              \
    J.r = r; J.w = w; J.k = k; J.v = v; J.kappa = kappa; J.a = a; J.s0 = s0;              \
    J.y = y; J.s_out = s_out; J.B = B; J.T = T; J.H = H; J.N = N;                         \
    J.ln_w = ln_w; J.ln_b = ln_b; J.r_k = r_k; J.eps = eps; J.epilogue = epilogue;        \
    return run(&J, nthreads, FN);                                                         \
}

/* Oracle proper: every operation in IEEE double. */
DEFINE_ENTRY(wkv7_oracle_forward_f64, double, run_head_f64)
/* fp32 twin (same loops in float): shows the floor of an fp32 evaluation. */
DEFINE_ENTRY(wkv7_oracle_forward_f32, float, run_head_f32)
