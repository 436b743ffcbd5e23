/*
 * csa_oracle.c -- plain CPU oracle for the CSA lightning-indexer top-k step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or helper with the HIP library; it is the slow, obviously-correct
 * definition that the GPU path is checked against.
 *
 * What it computes (StreamIndex: Memory-Bounded Compressed Sparse Attention
 * via Streaming Top-k, Abstract): every query position rates each compressed key
 * with the lightning indexer and keeps its k best keys.  The scoring rule
 * used throughout is
 *
 *     I(t, s) = sum_j  w[t, j] * max(0, q[t, j, :] . k[s, :])
 *
 * over the H indexer heads j, for the causally visible compressed keys s of
 * query position t.  With compression ratio m, key s summarises positions
 * s*m .. s*m+m-1, so it is visible to t exactly when (s+1)*m - 1 <= t, i.e.
 * the visible keys are the prefix s < n_vis(t) = min(T, floor((t+1)/m)).
 *
 * For fp8 inputs each row carries a positive fp32 scale; the dequantised
 * operands are q_scale[t,j]*q8[t,j,:] and k_scale[s]*k8[s,:], so the dot
 * product becomes q_scale[t,j]*k_scale[s]*(q8 . k8).
 *
 * Selection: all visible scores are sorted by (score descending, key index
 * ascending) and the first min(k, n_vis) are returned; the remaining slots
 * hold index -1 and score -infinity.  Ties go to the lower key index.
 *
 * Arithmetic: every input is decoded exactly to double and every sum is
 * taken in double, in plain loop order.  Output scores are doubles.
 *
 * A second mode (chunk > 0) runs the partition-merge form the abstract
 * describes: top-k of each chunk of `chunk` keys, concatenated, then top-k of
 * the concatenation.  It must equal the plain mode; tests check that.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_BF16 = 0, OR_E4M3FN = 1, OR_F32 = 2 };

/* ---------------------------------------------------------------- decoding */

/* bfloat16 is the upper 16 bits of an IEEE-754 binary32 word. */
double csa_oracle_decode_bf16(uint16_t bits)
{
    uint32_t word = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &word, sizeof f);
    return (double)f;
}

/* OCP 8-bit E4M3 ("fn": finite-only).  1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6;
 * exponent 15 with mantissa 7 is NaN; there is no infinity (FP8 Formats for
 * Deep Learning, section on the E4M3 encoding). */
double csa_oracle_decode_e4m3fn(uint8_t bits)
{
    int sign = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int mant = bits & 0x7;
    double v;
    if (e == 0xF && mant == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)mant / 8.0, -6);
    else
        v = ldexp(1.0 + (double)mant / 8.0, e - 7);
    return sign ? -v : v;
}

static double decode(const void *base, int dtype, int64_t i)
{
    switch (dtype) {
    case OR_BF16:
        return csa_oracle_decode_bf16(((const uint16_t *)base)[i]);
    case OR_E4M3FN:
        return csa_oracle_decode_e4m3fn(((const uint8_t *)base)[i]);
    default:
        return (double)((const float *)base)[i];
    }
}

/* ---------------------------------------------------------------- problem */

typedef struct {
    const void *q;         /* [nrows, H, D] query rows, one per requested t */
    int q_dtype;
    const float *q_scale;  /* [nrows, H] or NULL (= 1) */
    const float *w;        /* [nrows, H] */
    const void *k;         /* [T, D] compressed keys */
    int k_dtype;
    const float *k_scale;  /* [T] or NULL (= 1) */
    const int64_t *t;      /* [nrows] query positions */
    int64_t nrows, T;
    int H, D, m, topk;
    int64_t chunk;
    int32_t *out_idx;      /* [nrows, topk] */
    double *out_score;     /* [nrows, topk] */
    const double *kd;      /* [T, D] keys decoded to double */
} problem;

typedef struct {
    double score;
    int32_t idx;
} entry;

/* Order used for selection: larger score first, then smaller key index. */
static int cmp_entry(const void *pa, const void *pb)
{
    const entry *a = (const entry *)pa, *b = (const entry *)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    if (a->idx < b->idx) return -1;
    if (a->idx > b->idx) return 1;
    return 0;
}

int64_t csa_oracle_n_visible(int64_t t, int64_t T, int m)
{
    /* key s is visible iff (s+1)*m - 1 <= t  <=>  s < floor((t+1)/m) */
    int64_t n = (t + 1) / m;
    if (n < 0) n = 0;
    return n < T ? n : T;
}

/* Decode query row r to double: qd[j*D + x] = q[r, j, x]. */
static void decode_q_row(const problem *p, int64_t r, double *qd)
{
    for (int64_t i = 0; i < (int64_t)p->H * p->D; i++)
        qd[i] = decode(p->q, p->q_dtype, r * p->H * (int64_t)p->D + i);
}

/* Score of one (row, key) pair, straight from the definition.  qd is the
 * decoded query row r, kd the decoded key row s (k_scale not yet applied). */
static double score_pair(const problem *p, int64_t r, int64_t s,
                         const double *qd, const double *kd)
{
    double total = 0.0;
    double ks = p->k_scale ? (double)p->k_scale[s] : 1.0;
    for (int j = 0; j < p->H; j++) {
        double dot = 0.0;
        for (int x = 0; x < p->D; x++)
            dot += qd[j * p->D + x] * kd[x];
        double qs = p->q_scale ? (double)p->q_scale[r * p->H + j] : 1.0;
        double a = qs * ks * dot;
        double relu = a > 0.0 ? a : 0.0;
        total += (double)p->w[r * p->H + j] * relu;
    }
    return total;
}

/* Top-k of cand[0..n) under cmp_entry; result in cand[0..min(k,n)). */
static int64_t take_topk(entry *cand, int64_t n, int topk)
{
    qsort(cand, (size_t)n, sizeof(entry), cmp_entry);
    return n < topk ? n : topk;
}

static void solve_row(const problem *p, int64_t r, entry *buf, entry *merged,
                      double *qd)
{
    int64_t n = csa_oracle_n_visible(p->t[r], p->T, p->m);
    int64_t kept;
    decode_q_row(p, r, qd);
    for (int64_t s = 0; s < n; s++) {
        buf[s].score = score_pair(p, r, s, qd, p->kd + s * p->D);
        buf[s].idx = (int32_t)s;
    }
    if (p->chunk <= 0) {
        kept = take_topk(buf, n, p->topk);
        memcpy(merged, buf, (size_t)kept * sizeof(entry));
    } else {
        /* partition: top-k within each chunk; merge: top-k of the union */
        int64_t nm = 0;
        for (int64_t c0 = 0; c0 < n; c0 += p->chunk) {
            int64_t len = n - c0 < p->chunk ? n - c0 : p->chunk;
            int64_t got = take_topk(buf + c0, len, p->topk);
            memcpy(merged + nm, buf + c0, (size_t)got * sizeof(entry));
            nm += got;
        }
        kept = take_topk(merged, nm, p->topk);
    }
    for (int i = 0; i < p->topk; i++) {
        int64_t o = r * p->topk + i;
        if (i < kept) {
            p->out_idx[o] = merged[i].idx;
            p->out_score[o] = merged[i].score;
        } else {
            p->out_idx[o] = -1;
            p->out_score[o] = -INFINITY;
        }
    }
}

typedef struct {
    const problem *p;
    int64_t first, stride;  /* rows first, first+stride, ... */
    int status;
} job;

static void *run_job(void *arg)
{
    job *jb = (job *)arg;
    const problem *p = jb->p;
    entry *buf = (entry *)malloc((size_t)(p->T > 0 ? p->T : 1) * sizeof(entry));
    entry *merged = (entry *)malloc((size_t)(p->T > 0 ? p->T : 1) * sizeof(entry));
    double *qd = (double *)malloc((size_t)p->H * p->D * sizeof(double));
    if (!buf || !merged || !qd) {
        free(buf);
        free(merged);
        free(qd);
        jb->status = -1;
        return NULL;
    }
    for (int64_t r = jb->first; r < p->nrows; r += jb->stride)
        solve_row(p, r, buf, merged, qd);
    free(buf);
    free(merged);
    free(qd);
    jb->status = 0;
    return NULL;
}

/*
 * Top-k for `nrows` query rows.  q/q_scale/w hold only the requested rows
 * (row r belongs to position t[r]); k/k_scale hold all T keys of the batch.
 * Returns 0 on success, -1 on bad arguments or allocation failure.
 */
int csa_oracle_rows(const void *q, int q_dtype, const float *q_scale,
                    const float *w, const void *k, int k_dtype,
                    const float *k_scale, const int64_t *t, int64_t nrows,
                    int64_t T, int H, int D, int m, int topk, int64_t chunk,
                    int nthreads, int32_t *out_idx, double *out_score)
{
    if (!q || !w || !k || !t || !out_idx || !out_score) return -1;
    if (nrows < 0 || T < 0 || H < 1 || D < 1 || m < 1 || topk < 1) return -1;
    double *kd = (double *)malloc((size_t)(T > 0 ? T : 1) * D * sizeof(double));
    if (!kd) return -1;
    for (int64_t i = 0; i < T * D; i++)
        kd[i] = decode(k, k_dtype, i);
    problem p = {q, q_dtype, q_scale, w, k, k_dtype, k_scale, t, nrows, T,
                 H, D, m, topk, chunk, out_idx, out_score, kd};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = nrows > 0 ? (int)nrows : 1;
    job *jobs = (job *)calloc((size_t)nthreads, sizeof(job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        free(kd);
        return -1;
    }
    /* rows are dealt round-robin: cost grows with t, so this evens it out */
    int status = 0;
    for (int i = 0; i < nthreads; i++) {
        jobs[i].p = &p;
        jobs[i].first = i;
        jobs[i].stride = nthreads;
        if (pthread_create(&th[i], NULL, run_job, &jobs[i]) != 0) {
            run_job(&jobs[i]);
            th[i] = 0;
        }
    }
    for (int i = 0; i < nthreads; i++) {
        if (th[i]) pthread_join(th[i], NULL);
        if (jobs[i].status != 0) status = -1;
    }
    free(jobs);
    free(th);
    free(kd);
    return status;
}

/*
 * Scores of arbitrary (row, key) pairs, ignoring visibility.  Used by the
 * checker to score keys that a tested output returned but the oracle did not.
 */
int csa_oracle_score_pairs(const void *q, int q_dtype, const float *q_scale,
                           const float *w, const void *k, int k_dtype,
                           const float *k_scale, int64_t T, int H, int D,
                           const int64_t *row, const int64_t *key,
                           int64_t npairs, double *out)
{
    if (!q || !w || !k || !row || !key || !out || H < 1 || D < 1) return -1;
    problem p = {q, q_dtype, q_scale, w, k, k_dtype, k_scale, NULL, 0, T,
                 H, D, 1, 1, 0, NULL, NULL, NULL};
    double *qd = (double *)malloc((size_t)H * D * sizeof(double));
    double *kd = (double *)malloc((size_t)D * sizeof(double));
    if (!qd || !kd) {
        free(qd);
        free(kd);
        return -1;
    }
    int status = 0;
    for (int64_t i = 0; i < npairs; i++) {
        if (key[i] < 0 || key[i] >= T) {
            status = -1;
            break;
        }
        decode_q_row(&p, row[i], qd);
        for (int x = 0; x < D; x++)
            kd[x] = decode(k, k_dtype, key[i] * (int64_t)D + x);
        out[i] = score_pair(&p, row[i], key[i], qd, kd);
    }
    free(qd);
    free(kd);
    return status;
}
