/*
 * la_oracle.c -- plain, slow CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Everything is computed in fp64 with plain loops, in the order the pages
 * state the method.  Sources (page title, then section):
 *
 *   [Tut]  "六十四：MiniMax-01" (LLM tutorial, lesson 64), section 3
 *          "Lightning Attention 的定位": kernel-feature similarity
 *          phi(q)^T phi(k); the normalised causal output over i <= t; the
 *          recurrent state S_t = S_{t-1} + phi(k_t) v_t^T and normaliser
 *          z_t = z_{t-1} + phi(k_t); a new token needs only phi(q_t), S_t, z_t.
 *   [Arch] "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.1:
 *          Q, K, V = SiLU(.), Y = Q (K^T V), output RMSNorm(Y) * sigmoid(X).
 *
 * Readings where the pages are silent or garbled (each one is listed in the
 * design notes of the repository):
 *   - phi = SiLU, applied to q, k AND v ([Arch] 2.1 featurises all three;
 *     [Tut] 3 writes phi(k) v^T, we follow [Arch]).
 *   - the causal sum includes the current token (i <= t in [Tut] 3), so the
 *     state is updated with token t before y_t is read from it.
 *   - no 1/sqrt(d) scale and no decay (neither appears in the linear form).
 *   - default output y_t = phi(q_t)^T S_t ([Arch] 2.1 has no denominator);
 *     the normalised mode divides by phi(q_t)^T z_t ([Tut] 3), with no epsilon.
 *   - RMSNorm is per token over a group of features (default all H*d of the
 *     token), eps inside the square root, then times weight w, then times
 *     sigmoid(x) elementwise.
 *
 * The `flags` argument of every entry point: bit 0 (LAO_NORMALIZED) selects
 * the normalised output; bit 1 (LAO_FEATURES_GIVEN) says that q, k and v are
 * already feature vectors phi(.) -- the feature map applied by whoever
 * produced them, e.g. in the epilogue of the projection that computes them
 * ([Arch] 2.1 writes Q, K, V = SiLU(X W)) -- so it is not applied again here.
 *
 * Functions return 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double silu(double x) { return x / (1.0 + exp(-x)); }
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

enum { LAO_NORMALIZED = 1, LAO_FEATURES_GIVEN = 2 };

/* The feature map phi of one input value under `flags`. */
static double feature(double x, int flags) { return (flags & LAO_FEATURES_GIVEN) ? x : silu(x); }

/* One token of the recurrence for one (sequence, head) pair, in place.
 * [Tut] 3: S <- S + phi(k) phi(v)^T, z <- z + phi(k); then
 * y = phi(q)^T S, optionally divided by phi(q)^T z.
 * S is d x d row-major, S[i*d + j] pairs key feature i with value feature j. */
static void recurrent_token(const double* qt, const double* kt, const double* vt,
                            int d, int flags, double* S, double* z,
                            double* a, double* b, double* c, double* yt)
{
    for (int i = 0; i < d; i++) {
        a[i] = feature(qt[i], flags);
        b[i] = feature(kt[i], flags);
        c[i] = feature(vt[i], flags);
    }
    for (int i = 0; i < d; i++)
        for (int j = 0; j < d; j++)
            S[(size_t)i * d + j] += b[i] * c[j];
    if (flags & LAO_NORMALIZED)
        for (int i = 0; i < d; i++) z[i] += b[i];
    if (!yt) return;
    for (int j = 0; j < d; j++) {
        double acc = 0.0;
        for (int i = 0; i < d; i++) acc += a[i] * S[(size_t)i * d + j];
        yt[j] = acc;
    }
    if (flags & LAO_NORMALIZED) {
        double den = 0.0;
        for (int i = 0; i < d; i++) den += a[i] * z[i];
        for (int j = 0; j < d; j++) yt[j] /= den;
    }
}

/* ------------------------------------------------------------------------ */
/* Thread pool over (sequence, head) pairs.                                 */

typedef struct {
    const double *q, *k, *v;
    const float *qf, *kf, *vf;  /* float inputs (widened exactly) instead of q, k, v */
    const int64_t* cu;
    int32_t nseq, H, d, flags;
    const double *state_in, *z_in;
    double *y, *state_out, *z_out;
    const int64_t* sample_idx; /* sorted global token indices, or NULL */
    int64_t nsample;
    int32_t nthreads;
    int32_t block;             /* 0: recurrent form; >0: blocked form with this block */
    int32_t fp32;              /* blocked form only: do the arithmetic in float */
} job_t;

typedef struct { job_t* job; int32_t tid; int32_t status; } worker_t;

static int64_t lower_bound(const int64_t* a, int64_t n, int64_t x)
{
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (a[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo;
}

static int run_pair_recurrent(job_t* J, int32_t s, int32_t h)
{
    const int d = J->d, H = J->H;
    double* S = (double*)calloc((size_t)d * d, sizeof(double));
    double* z = (double*)calloc((size_t)d, sizeof(double));
    double* a = (double*)malloc((size_t)d * sizeof(double));
    double* b = (double*)malloc((size_t)d * sizeof(double));
    double* c = (double*)malloc((size_t)d * sizeof(double));
    double* yt = (double*)malloc((size_t)d * sizeof(double));
    double* qt = (double*)malloc((size_t)3 * d * sizeof(double));
    if (!S || !z || !a || !b || !c || !yt || !qt) {
        free(S); free(z); free(a); free(b); free(c); free(yt); free(qt);
        return -1;
    }
    double* kt = qt + d;
    double* vt = qt + 2 * d;
    if (J->state_in)
        memcpy(S, J->state_in + ((size_t)s * H + h) * d * d, (size_t)d * d * sizeof(double));
    if (J->z_in)
        memcpy(z, J->z_in + ((size_t)s * H + h) * d, (size_t)d * sizeof(double));

    const int64_t t0 = J->cu[s], t1 = J->cu[s + 1];
    int64_t si = J->sample_idx ? lower_bound(J->sample_idx, J->nsample, t0) : 0;
    for (int64_t t = t0; t < t1; t++) {
        const size_t off = ((size_t)t * H + h) * d;
        double* dst = NULL;
        if (!J->sample_idx) {
            dst = J->y + off;
        } else if (si < J->nsample && J->sample_idx[si] == t) {
            dst = yt;
        }
        if (J->qf) {
            for (int i = 0; i < d; i++) {
                qt[i] = (double)J->qf[off + i];
                kt[i] = (double)J->kf[off + i];
                vt[i] = (double)J->vf[off + i];
            }
            recurrent_token(qt, kt, vt, d, J->flags, S, z, a, b, c, dst);
        } else {
            recurrent_token(J->q + off, J->k + off, J->v + off, d, J->flags, S, z, a, b, c, dst);
        }
        if (J->sample_idx && dst) {
            /* several equal sample indices all receive this token's output */
            while (si < J->nsample && J->sample_idx[si] == t) {
                memcpy(J->y + ((size_t)si * H + h) * d, yt, (size_t)d * sizeof(double));
                si++;
            }
        }
    }
    if (J->state_out)
        memcpy(J->state_out + ((size_t)s * H + h) * d * d, S, (size_t)d * d * sizeof(double));
    if (J->z_out)
        memcpy(J->z_out + ((size_t)s * H + h) * d, z, (size_t)d * sizeof(double));
    free(S); free(z); free(a); free(b); free(c); free(yt); free(qt);
    return 0;
}

/* Blocked form of the same sum, written as the pages' blocked method does it:
 * within a block of B tokens the masked quadratic form (phi(Q) phi(K)^T (.) M) phi(V)
 * with M[t][i] = 1 iff i <= t; across blocks the state carried from the
 * previous blocks, phi(Q) S_prev; after the block S += phi(K)^T phi(V).
 * ([Arch] 2.1 gives Q (K^T V) for the inter-block part; [Tut] 3 the causal
 * sum.)  Used only to check that the recurrence is block-size invariant, in
 * double or in float arithmetic. */
#define BLOCKED_BODY(T_)                                                            \
    do {                                                                            \
        T_* S = (T_*)calloc((size_t)d * d, sizeof(T_));                             \
        T_* z = (T_*)calloc((size_t)d, sizeof(T_));                                 \
        T_* fq = (T_*)malloc((size_t)B * d * sizeof(T_));                           \
        T_* fk = (T_*)malloc((size_t)B * d * sizeof(T_));                           \
        T_* fv = (T_*)malloc((size_t)B * d * sizeof(T_));                           \
        T_* P = (T_*)malloc((size_t)B * B * sizeof(T_));                            \
        if (!S || !z || !fq || !fk || !fv || !P) {                                  \
            free(S); free(z); free(fq); free(fk); free(fv); free(P);                \
            return -1;                                                              \
        }                                                                           \
        if (J->state_in)                                                            \
            for (size_t e = 0; e < (size_t)d * d; e++)                              \
                S[e] = (T_)J->state_in[((size_t)s * H + h) * d * d + e];            \
        if (J->z_in)                                                                \
            for (int e = 0; e < d; e++) z[e] = (T_)J->z_in[((size_t)s * H + h) * d + e]; \
        for (int64_t b0 = t0; b0 < t1; b0 += B) {                                   \
            const int n = (int)((t1 - b0) < B ? (t1 - b0) : B);                     \
            for (int r = 0; r < n; r++)                                             \
                for (int e = 0; e < d; e++) {                                       \
                    const size_t off = ((size_t)(b0 + r) * H + h) * d + e;          \
                    fq[r * d + e] = (T_)feature(J->q[off], J->flags);               \
                    fk[r * d + e] = (T_)feature(J->k[off], J->flags);               \
                    fv[r * d + e] = (T_)feature(J->v[off], J->flags);               \
                }                                                                   \
            for (int r = 0; r < n; r++)                                             \
                for (int c2 = 0; c2 < n; c2++) {                                    \
                    T_ acc = 0;                                                     \
                    if (c2 <= r)                                                    \
                        for (int e = 0; e < d; e++) acc += fq[r * d + e] * fk[c2 * d + e]; \
                    P[r * B + c2] = acc;                                            \
                }                                                                   \
            for (int r = 0; r < n; r++) {                                           \
                double* yr = J->y + ((size_t)(b0 + r) * H + h) * d;                 \
                T_ den = 0;                                                         \
                if (J->flags & LAO_NORMALIZED) {                                                \
                    for (int c2 = 0; c2 <= r; c2++) den += P[r * B + c2];           \
                    for (int e = 0; e < d; e++) den += fq[r * d + e] * z[e];        \
                }                                                                   \
                for (int j = 0; j < d; j++) {                                       \
                    T_ intra = 0, inter = 0;                                        \
                    for (int c2 = 0; c2 <= r; c2++) intra += P[r * B + c2] * fv[c2 * d + j]; \
                    for (int i = 0; i < d; i++) inter += fq[r * d + i] * S[(size_t)i * d + j]; \
                    T_ yv = intra + inter;                                          \
                    if (J->flags & LAO_NORMALIZED) yv /= den;                                   \
                    yr[j] = (double)yv;                                             \
                }                                                                   \
            }                                                                       \
            for (int i = 0; i < d; i++)                                             \
                for (int j = 0; j < d; j++) {                                       \
                    T_ acc = 0;                                                     \
                    for (int r = 0; r < n; r++) acc += fk[r * d + i] * fv[r * d + j]; \
                    S[(size_t)i * d + j] += acc;                                    \
                }                                                                   \
            if (J->flags & LAO_NORMALIZED)                                                      \
                for (int i = 0; i < d; i++) {                                       \
                    T_ acc = 0;                                                     \
                    for (int r = 0; r < n; r++) acc += fk[r * d + i];               \
                    z[i] += acc;                                                    \
                }                                                                   \
        }                                                                           \
        if (J->state_out)                                                           \
            for (size_t e = 0; e < (size_t)d * d; e++)                              \
                J->state_out[((size_t)s * H + h) * d * d + e] = (double)S[e];       \
        if (J->z_out)                                                               \
            for (int e = 0; e < d; e++) J->z_out[((size_t)s * H + h) * d + e] = (double)z[e]; \
        free(S); free(z); free(fq); free(fk); free(fv); free(P);                    \
    } while (0)

static int run_pair_blocked(job_t* J, int32_t s, int32_t h)
{
    const int d = J->d, H = J->H, B = J->block;
    const int64_t t0 = J->cu[s], t1 = J->cu[s + 1];
    if (J->fp32) BLOCKED_BODY(float);
    else BLOCKED_BODY(double);
    return 0;
}

static void* worker_main(void* arg)
{
    worker_t* W = (worker_t*)arg;
    job_t* J = W->job;
    const int64_t pairs = (int64_t)J->nseq * J->H;
    W->status = 0;
    for (int64_t p = W->tid; p < pairs; p += J->nthreads) {
        const int32_t s = (int32_t)(p / J->H), h = (int32_t)(p % J->H);
        const int rc = J->block > 0 ? run_pair_blocked(J, s, h) : run_pair_recurrent(J, s, h);
        if (rc) W->status = rc;
    }
    return NULL;
}

static int run_job(job_t* J)
{
    int32_t nt = J->nthreads;
    const int64_t pairs = (int64_t)J->nseq * J->H;
    if (nt < 1) nt = 1;
    if (nt > pairs) nt = (int32_t)(pairs > 0 ? pairs : 1);
    J->nthreads = nt;
    worker_t* W = (worker_t*)calloc((size_t)nt, sizeof(worker_t));
    pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    if (!W || !th) { free(W); free(th); return -1; }
    int status = 0;
    for (int i = 0; i < nt; i++) {
        W[i].job = J; W[i].tid = i;
        if (i > 0 && pthread_create(&th[i], NULL, worker_main, &W[i]) != 0) {
            worker_main(&W[i]);
            th[i] = 0;
        }
    }
    worker_main(&W[0]);
    for (int i = 1; i < nt; i++)
        if (th[i]) pthread_join(th[i], NULL);
    for (int i = 0; i < nt; i++)
        if (W[i].status) status = W[i].status;
    free(W); free(th);
    return status;
}

static int check_cu(const int64_t* cu, int32_t nseq)
{
    if (!cu || nseq < 1 || cu[0] != 0) return -1;
    for (int32_t s = 0; s < nseq; s++)
        if (cu[s + 1] < cu[s]) return -1;
    return 0;
}

/* Recurrent form over a packed batch.
 * q, k, v: [total_T, H, d] pre-activation values (fp64).
 * cu_seqlens: [nseq + 1] token offsets, cu[0] = 0, non-decreasing.
 * state_in [nseq, H, d, d], z_in [nseq, H, d]: initial state or NULL (zeros).
 * y: [total_T, H, d] if sample_idx is NULL, else [nsample, H, d] holding the
 *    outputs of the listed global tokens (sample_idx sorted ascending).
 * state_out, z_out: final state per (sequence, head) or NULL. */
int lao_prefill(const double* q, const double* k, const double* v,
                const int64_t* cu_seqlens, int32_t nseq, int32_t H, int32_t d,
                const double* state_in, const double* z_in, int32_t flags,
                double* y, double* state_out, double* z_out,
                const int64_t* sample_idx, int64_t nsample, int32_t nthreads)
{
    if (!q || !k || !v || !y || H < 1 || d < 1 || check_cu(cu_seqlens, nseq)) return -1;
    if (sample_idx) {
        for (int64_t i = 0; i < nsample; i++) {
            if (sample_idx[i] < 0 || sample_idx[i] >= cu_seqlens[nseq]) return -1;
            if (i && sample_idx[i] < sample_idx[i - 1]) return -1;
        }
    }
    job_t J = {q, k, v, NULL, NULL, NULL, cu_seqlens, nseq, H, d, flags, state_in, z_in,
               y, state_out, z_out, sample_idx, nsample, nthreads, 0, 0};
    return run_job(&J);
}

/* Same as lao_prefill with float inputs (bf16 or fp32 values), each widened
 * exactly to double as it is used: for inputs too large to hold in double. */
int lao_prefill_f32in(const float* q, const float* k, const float* v,
                      const int64_t* cu_seqlens, int32_t nseq, int32_t H, int32_t d,
                      const double* state_in, const double* z_in, int32_t flags,
                      double* y, double* state_out, double* z_out,
                      const int64_t* sample_idx, int64_t nsample, int32_t nthreads)
{
    if (!q || !k || !v || !y || H < 1 || d < 1 || check_cu(cu_seqlens, nseq)) return -1;
    if (sample_idx) {
        for (int64_t i = 0; i < nsample; i++) {
            if (sample_idx[i] < 0 || sample_idx[i] >= cu_seqlens[nseq]) return -1;
            if (i && sample_idx[i] < sample_idx[i - 1]) return -1;
        }
    }
    job_t J = {NULL, NULL, NULL, q, k, v, cu_seqlens, nseq, H, d, flags, state_in, z_in,
               y, state_out, z_out, sample_idx, nsample, nthreads, 0, 0};
    return run_job(&J);
}

/* Blocked form (block > 0), in double (fp32 == 0) or float (fp32 == 1);
 * same arguments as lao_prefill without sampling. */
int lao_prefill_blocked(const double* q, const double* k, const double* v,
                        const int64_t* cu_seqlens, int32_t nseq, int32_t H, int32_t d,
                        const double* state_in, const double* z_in, int32_t flags,
                        double* y, double* state_out, double* z_out,
                        int32_t block, int32_t fp32, int32_t nthreads)
{
    if (!q || !k || !v || !y || H < 1 || d < 1 || block < 1 || check_cu(cu_seqlens, nseq)) return -1;
    job_t J = {q, k, v, NULL, NULL, NULL, cu_seqlens, nseq, H, d, flags, state_in, z_in,
               y, state_out, z_out, NULL, 0, nthreads, block, fp32 ? 1 : 0};
    return run_job(&J);
}

/* One decode step for N independent sequences ([Tut] 3: a new token only
 * updates S and z and reads its output from them).
 * q, k, v, y: [N, H, d]; S: [N, H, d, d] and z: [N, H, d] updated in place. */
int lao_decode_step(const double* q, const double* k, const double* v,
                    int32_t N, int32_t H, int32_t d, int32_t flags,
                    double* S, double* z, double* y)
{
    if (!q || !k || !v || !S || !y || ((flags & LAO_NORMALIZED) && !z) || N < 0 || H < 1 || d < 1)
        return -1;
    double* a = (double*)malloc((size_t)d * sizeof(double));
    double* b = (double*)malloc((size_t)d * sizeof(double));
    double* c = (double*)malloc((size_t)d * sizeof(double));
    double* zdummy = (double*)calloc((size_t)d, sizeof(double));
    if (!a || !b || !c || !zdummy) { free(a); free(b); free(c); free(zdummy); return -1; }
    for (int64_t p = 0; p < (int64_t)N * H; p++) {
        const size_t off = (size_t)p * d;
        recurrent_token(q + off, k + off, v + off, d, flags, S + (size_t)p * d * d,
                        (flags & LAO_NORMALIZED) ? z + off : zdummy, a, b, c, y + off);
    }
    free(a); free(b); free(c); free(zdummy);
    return 0;
}

/* Output gate of [Arch] 2.1: per token, RMSNorm over groups of `group`
 * consecutive features of Y (F features per token, F % group == 0),
 *   r = 1 / sqrt(mean(Y_g^2) + eps),  out = Y * r * w * sigmoid(x).
 * y, x, out: [ntok, F]; w: [F] or NULL (unit weight). */
int lao_gate(const double* y, const double* x, const double* w, int64_t ntok,
             int32_t F, int32_t group, double eps, double* out)
{
    if (!y || !x || !out || F < 1 || group < 1 || F % group) return -1;
    for (int64_t t = 0; t < ntok; t++) {
        const double* yt = y + (size_t)t * F;
        const double* xt = x + (size_t)t * F;
        double* ot = out + (size_t)t * F;
        for (int32_t g0 = 0; g0 < F; g0 += group) {
            double ss = 0.0;
            for (int32_t f = g0; f < g0 + group; f++) ss += yt[f] * yt[f];
            const double r = 1.0 / sqrt(ss / group + eps);
            for (int32_t f = g0; f < g0 + group; f++)
                ot[f] = yt[f] * r * (w ? w[f] : 1.0) * sigmoid(xt[f]);
        }
    }
    return 0;
}
