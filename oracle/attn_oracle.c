/*
 * attn_oracle.c -- plain, slow fp64 CPU oracle for causal GQA prefill attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * library (it is built with gcc, not hipcc).
 *
 * What it computes (the plain definition; no tiling, no online softmax):
 *   "Why Attention Scaling Breaks", section "The O(n^2) problem": scores
 *   S = Q K^T, weights A = softmax(S / sqrt(d)), output O = A V, with the
 *   whole score row materialised.
 *   "Long-Context Attention Explained", sections on quadratic cost: with a
 *   causal model each token looks only backwards, itself included, so query i
 *   sees keys j <= i.  The safe-softmax step subtracts the row maximum before
 *   exponentiating (section "Online softmax", closing remark, and the naive
 *   NumPy routine in the teaching code).
 *   "flops / prefill-attention", section "Arithmetic intensity": n_q query
 *   heads share n_kv key/value heads (group ratio g = n_q / n_kv); the causal
 *   flop count is 2 * n_q * d_h * L^2 per sequence.
 *   "Long-Context Attention Explained", section "What FlashAttention does not
 *   change": the backward pass needs small saved row statistics; this oracle
 *   emits that statistic as the natural-log log-sum-exp of the scaled scores,
 *   LSE = m + ln(sum_j exp(s_j - m)).
 *
 * Readings where the pages are silent (each is listed with its reason in the
 * design notes): query head h reads key/value head floor(h / g); the scale is
 * the caller's fp32 value, widened exactly; inputs are bf16 bit patterns,
 * widened exactly to fp64; everything after that is fp64.
 *
 * Chunked prefill ("flops / prefill-attention", section "Workarounds": a long
 * prompt split into pieces): a chunk of Lq queries against Lk keys, query
 * row i sitting at key position q_off + i, so that causally it sees keys
 * j <= q_off + i.  With Lq = Lk = L and q_off = 0 this is the whole-sequence
 * case above.
 *
 * Layouts: q [B, n_q, Lq, d_h], k and v [B, n_kv, Lk, d_h], all bf16 bit
 * patterns (uint16), row-major, d_h fastest.  A "row" is the flat index
 * (b * n_q + h) * Lq + i of one query.
 *
 * Parity pins: every function here is pinned by CPU tests against brute force
 * in 50-digit arithmetic, closed forms and a library routine; nothing in it is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

int oracle_version(void) { return 2; }

/* A bf16 bit pattern is the upper half of an fp32 bit pattern, so widening is
 * exact: shift into place, reinterpret as float, convert to double. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One query row, done the plain way.  s and w are scratch rows of length Lk. */
static void one_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                    int64_t Lq, int64_t Lk, int64_t q_off, int64_t n_q,
                    int64_t n_kv, int64_t d_h, double scale, int causal,
                    int64_t row, double *s, double *w, double *out,
                    double *lse, uint64_t *flops)
{
    const int64_t L = Lk;
    const int64_t g = n_q / n_kv;
    const int64_t i = row % Lq;
    const int64_t h = (row / Lq) % n_q;
    const int64_t b = row / (Lq * n_q);
    const int64_t kvh = h / g;
    const uint16_t *qrow = q + ((b * n_q + h) * Lq + i) * d_h;
    const uint16_t *kbase = k + (b * n_kv + kvh) * Lk * d_h;
    const uint16_t *vbase = v + (b * n_kv + kvh) * Lk * d_h;
    /* visible keys: j <= q_off + i when causal, all Lk keys otherwise */
    const int64_t n_vis = causal ? q_off + i + 1 : Lk;

    /* 1. materialise the whole score row; masked entries are -inf and their
     *    dot products are never formed */
    for (int64_t j = 0; j < L; ++j) {
        if (j < n_vis) {
            const uint16_t *krow = kbase + j * d_h;
            double dot = 0.0;
            for (int64_t t = 0; t < d_h; ++t)
                dot += widen_bf16(qrow[t]) * widen_bf16(krow[t]);
            s[j] = scale * dot;
        } else {
            s[j] = -INFINITY;
        }
    }
    /* 2. row maximum (safe softmax) */
    double m = -INFINITY;
    for (int64_t j = 0; j < L; ++j)
        if (s[j] > m) m = s[j];
    /* 3. exponentials and their plain sum; exp(-inf) = 0 for masked keys */
    double total = 0.0;
    for (int64_t j = 0; j < L; ++j) {
        w[j] = exp(s[j] - m);
        total += w[j];
    }
    /* 4. normalised weights P = w / total, materialised */
    for (int64_t j = 0; j < L; ++j)
        w[j] = w[j] / total;
    /* 5. O = P V over the visible keys (masked weights are exactly zero) */
    for (int64_t t = 0; t < d_h; ++t)
        out[t] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const uint16_t *vrow = vbase + j * d_h;
        const double p = w[j];
        for (int64_t t = 0; t < d_h; ++t)
            out[t] += p * widen_bf16(vrow[t]);
    }
    /* 6. saved row statistic: natural-log log-sum-exp of the scaled scores */
    *lse = m + log(total);
    /* 2*d_h flops per visible pair for Q K^T and 2*d_h for P V */
    *flops += (uint64_t)(4 * d_h * n_vis);
}

/*
 * Attention of a chunk for the requested rows.
 *   rows == NULL: every row, in flat order (n_rows must equal B*n_q*Lq).
 *   q_off >= 0, and q_off + Lq <= Lk when causal (every query sees its own
 *   position).
 *   out:  [n_rows, d_h] fp64, lse: [n_rows] fp64, flops: counted flops.
 *   threads <= 0 leaves the OpenMP default.
 * Returns ORACLE_OK, ORACLE_BAD_ARG or ORACLE_NO_MEMORY.
 */
int oracle_attn_rows_chunk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int64_t B, int64_t Lq, int64_t Lk, int64_t q_off,
                           int64_t n_q, int64_t n_kv, int64_t d_h, float scale,
                           int causal, const int64_t *rows, int64_t n_rows,
                           double *out, double *lse, uint64_t *flops, int threads)
{
    if (!q || !k || !v || !out || !lse || !flops) return ORACLE_BAD_ARG;
    if (B < 1 || Lq < 1 || Lk < 1 || n_q < 1 || n_kv < 1 || d_h < 1) return ORACLE_BAD_ARG;
    if (n_q % n_kv != 0) return ORACLE_BAD_ARG;
    if (causal != 0 && causal != 1) return ORACLE_BAD_ARG;
    if (q_off < 0 || (causal && q_off + Lq > Lk)) return ORACLE_BAD_ARG;
    if (!isfinite(scale)) return ORACLE_BAD_ARG;
    const int64_t total_rows = B * n_q * Lq;
    if (rows == NULL && n_rows != total_rows) return ORACLE_BAD_ARG;
    if (rows != NULL)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= total_rows) return ORACLE_BAD_ARG;

    const double sc = (double)scale;
    uint64_t count = 0;
    int failed = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel reduction(+ : count) reduction(| : failed)
    {
        double *s = (double *)malloc((size_t)Lk * sizeof(double));
        double *w = (double *)malloc((size_t)Lk * sizeof(double));
        /* every thread reaches the work-sharing loop, even one whose scratch
         * allocation failed; such a thread only records the failure */
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < n_rows; ++r) {
            if (!s || !w) {
                failed = 1;
                continue;
            }
            const int64_t row = rows ? rows[r] : r;
            one_row(q, k, v, Lq, Lk, q_off, n_q, n_kv, d_h, sc, causal, row, s, w,
                    out + r * d_h, lse + r, &count);
        }
        free(s);
        free(w);
    }
    *flops = count;
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/* Whole-sequence attention for the requested rows: the chunk with
 * Lq = Lk = L and q_off = 0 (rows are (b * n_q + h) * L + i). */
int oracle_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     int64_t B, int64_t L, int64_t n_q, int64_t n_kv,
                     int64_t d_h, float scale, int causal,
                     const int64_t *rows, int64_t n_rows,
                     double *out, double *lse, uint64_t *flops, int threads)
{
    return oracle_attn_rows_chunk(q, k, v, B, L, L, 0, n_q, n_kv, d_h, scale, causal,
                                  rows, n_rows, out, lse, flops, threads);
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
