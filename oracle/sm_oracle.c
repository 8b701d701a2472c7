/*
 * sm_oracle.c -- plain, slow CPU oracle for the softmax attention layer of
 * the hybrid model (the one layer in eight that is not linear attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * Everything is computed in fp64 with plain loops.  Sources (page title, then
 * section):
 *
 *   [Tut]  "六十四：MiniMax-01" (LLM tutorial, lesson 64), sections 2-3:
 *          the softmax layer computes softmax(Q K^T / sqrt(d)) V, with a
 *          cost quadratic in the sequence length.
 *   [Arch] "MiniMax-Text-01 405B MoE模型架构与训练策略解析", section 2.2: the
 *          softmax layers apply rotary position embedding to half of each
 *          head's dimensions, with base 10,000; section 4.1: the base is
 *          raised to 5M and then 10M for the long-context stages.
 *   [Overview] "MiniMax-01系列大模型：超长上下文与多模态能力深度解析与部署指南",
 *          section 2.1.3: variable-length (varlen) packing for the softmax
 *          layers (named with its ring communication across devices).
 *
 * Readings where the pages are silent (each one is listed in the design
 * notes of the repository):
 *   - causal: query t attends to keys u <= t of its own sequence (a language
 *     model layer); positions restart at 0 at each sequence start.
 *   - rotary pairs: inside the first `rot` dimensions, dimension j is paired
 *     with j + rot/2 (j < rot/2), rotated by the angle pos * base^(-2j/rot):
 *         x'_j        = x_j cos - x_{j+rot/2} sin
 *         x'_{j+rot/2} = x_{j+rot/2} cos + x_j sin
 *     dimensions rot .. d-1 are left as they are.  rot = d/2 is the pages'
 *     half; the interleaved pairing (2j, 2j+1) differs from this one by a
 *     fixed permutation of q's and k's features, which leaves every score
 *     unchanged when applied to both.
 *   - the score scale is 1/sqrt(d) unless the caller gives another one.
 *   - grouped heads: query head h reads key/value head h / (H / Hkv)
 *     (Hkv = H is plain multi-head attention).
 *   - lse = log sum_u exp(score_u), natural log, per (token, head).
 *
 * Functions return 0 on success, -1 on an invalid argument.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* [Arch] 2.2: rotary embedding of one head vector at position `pos`, on the
 * first `rot` dimensions; cs holds cos and sin of pos * theta_j, j < rot/2. */
static void rope(const double* x, const double* cs, int d, int rot, double* out)
{
    const int half = rot / 2;
    for (int j = 0; j < half; j++) {
        const double c = cs[2 * j], s = cs[2 * j + 1];
        out[j] = x[j] * c - x[j + half] * s;
        out[j + half] = x[j + half] * c + x[j] * s;
    }
    for (int j = rot; j < d; j++) out[j] = x[j];
}

typedef struct {
    const double *q, *k, *v;
    const int64_t* cu;
    int64_t nseq, H, Hkv, d, rot;
    double scale;
    const double* cs;     /* [max_len, rot/2, 2] cos/sin by position */
    const int64_t *rows, *heads;
    int64_t n;
    double *out, *lse;
    int64_t next;         /* work counter (pairs), under mu */
    pthread_mutex_t mu;
} sm_job_t;

static int64_t seq_of(const int64_t* cu, int64_t nseq, int64_t t)
{
    int64_t lo = 0, hi = nseq; /* largest s with cu[s] <= t < cu[s+1] */
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) / 2;
        if (cu[mid] <= t) lo = mid; else hi = mid;
    }
    while (lo + 1 < nseq && cu[lo + 1] <= t) lo++;
    return lo;
}

/* Output of one (token, query head) pair: [Tut] 2-3 softmax over the
 * scores of keys u <= t of the sequence, then the weighted sum of values. */
static void one_pair(sm_job_t* J, int64_t t, int64_t h, double* qr, double* kr, double* sc,
                     double* y, double* lse)
{
    const int64_t d = J->d, H = J->H, Hkv = J->Hkv, half = J->rot / 2;
    const int64_t s = seq_of(J->cu, J->nseq, t);
    const int64_t t0 = J->cu[s];
    const int64_t hk = h / (H / Hkv);
    rope(J->q + (t * H + h) * d, J->cs + (t - t0) * half * 2, (int)d, (int)J->rot, qr);
    double mx = -INFINITY;
    for (int64_t u = t0; u <= t; u++) {
        rope(J->k + (u * Hkv + hk) * d, J->cs + (u - t0) * half * 2, (int)d, (int)J->rot, kr);
        double dot = 0.0;
        for (int64_t j = 0; j < d; j++) dot += qr[j] * kr[j];
        sc[u - t0] = J->scale * dot;
        if (sc[u - t0] > mx) mx = sc[u - t0];
    }
    double den = 0.0;
    for (int64_t j = 0; j < d; j++) y[j] = 0.0;
    for (int64_t u = t0; u <= t; u++) {
        const double w = exp(sc[u - t0] - mx);
        den += w;
        const double* vu = J->v + (u * Hkv + hk) * d;
        for (int64_t j = 0; j < d; j++) y[j] += w * vu[j];
    }
    for (int64_t j = 0; j < d; j++) y[j] /= den;
    *lse = mx + log(den);
}

static void* sm_worker(void* arg)
{
    sm_job_t* J = (sm_job_t*)arg;
    int64_t maxlen = 0;
    for (int64_t s = 0; s < J->nseq; s++)
        if (J->cu[s + 1] - J->cu[s] > maxlen) maxlen = J->cu[s + 1] - J->cu[s];
    double* qr = malloc(sizeof(double) * J->d);
    double* kr = malloc(sizeof(double) * J->d);
    double* sc = malloc(sizeof(double) * (maxlen > 0 ? maxlen : 1));
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t i = J->next < J->n ? J->next++ : -1;
        pthread_mutex_unlock(&J->mu);
        if (i < 0) break;
        double l;
        one_pair(J, J->rows[i], J->heads[i], qr, kr, sc, J->out + i * J->d, &l);
        if (J->lse) J->lse[i] = l;
    }
    free(qr);
    free(kr);
    free(sc);
    return NULL;
}

/* Causal softmax attention with rotary embedding, at the listed
 * (token, query head) pairs.
 *   q [T, H, d], k and v [T, Hkv, d] (fp64); cu [nseq + 1] sequence starts
 *   (0 = cu[0] <= ... <= cu[nseq] = T); rot even in [0, d]; base > 0;
 *   scale > 0 (the caller passes 1/sqrt(d) for the pages' form);
 *   rows[i], heads[i]: pair i (rows in [0, T), heads in [0, H)), i < n;
 *   out [n, d]; lse [n] or NULL. */
int smo_attention(const double* q, const double* k, const double* v, const int64_t* cu,
                  int64_t nseq, int64_t H, int64_t Hkv, int64_t d, int64_t rot, double base,
                  double scale, const int64_t* rows, const int64_t* heads, int64_t n,
                  double* out, double* lse, int32_t nthreads)
{
    if (!q || !k || !v || !cu || nseq < 1 || H < 1 || Hkv < 1 || H % Hkv || d < 1 || rot < 0 ||
        rot > d || rot % 2 || !(base > 0.0) || !(scale > 0.0) || n < 0 || (n && (!rows || !heads || !out)))
        return -1;
    if (cu[0] != 0) return -1;
    for (int64_t s = 0; s < nseq; s++)
        if (cu[s + 1] < cu[s]) return -1;
    const int64_t T = cu[nseq];
    int64_t maxlen = 0;
    for (int64_t s = 0; s < nseq; s++)
        if (cu[s + 1] - cu[s] > maxlen) maxlen = cu[s + 1] - cu[s];
    for (int64_t i = 0; i < n; i++)
        if (rows[i] < 0 || rows[i] >= T || heads[i] < 0 || heads[i] >= H) return -1;

    /* [Arch] 2.2, 4.1: theta_j = base^(-2j/rot); cos and sin of pos * theta_j */
    const int64_t half = rot / 2;
    double* cs = malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1) * (half > 0 ? half : 1) * 2);
    if (!cs) return -1;
    for (int64_t j = 0; j < half; j++) {
        const double theta = pow(base, -2.0 * (double)j / (double)rot);
        for (int64_t p = 0; p < maxlen; p++) {
            cs[(p * half + j) * 2] = cos((double)p * theta);
            cs[(p * half + j) * 2 + 1] = sin((double)p * theta);
        }
    }

    sm_job_t J = {q, k, v, cu, nseq, H, Hkv, d, rot, scale, cs, rows, heads, n, out, lse, 0};
    pthread_mutex_init(&J.mu, NULL);
    int nt = nthreads > 0 ? nthreads : 1;
    if (nt > 64) nt = 64;
    pthread_t th[64];
    for (int i = 0; i < nt; i++) pthread_create(&th[i], NULL, sm_worker, &J);
    for (int i = 0; i < nt; i++) pthread_join(th[i], NULL);
    pthread_mutex_destroy(&J.mu);
    free(cs);
    return 0;
}
