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
 * Readings where the pages are silent: query head h reads key/value head
 * floor(h / g) (consecutive query heads form a group, the repeat-interleave
 * reading of heads sharing K and V); the scale is the caller's fp32 value,
 * widened exactly; inputs are bf16 bit patterns, widened exactly to fp64;
 * everything after that is fp64.
 *
 * Chunked prefill ("flops / prefill-attention", section "Workarounds": a long
 * prompt split into pieces): a chunk of Lq queries against Lk keys, query
 * row i sitting at key position q_off + i, so that causally it sees keys
 * j <= q_off + i.  With Lq = Lk = L and q_off = 0 this is the whole-sequence
 * case above.
 *
 * FP8 inputs ("flops / prefill-attention", section "Workarounds", FP8
 * attention): q, k, v may instead be OCP e4m3 codes with an fp32 descale
 * factor each; the oracle decodes every code exactly (sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, subnormals below 2^-6, S.1111.111 = NaN),
 * multiplies by the descale in fp64 and runs the same plain attention.
 *
 * Layouts: q [B, n_q, Lq, d_h], k and v [B, n_kv, Lk, d_h], bf16 bit
 * patterns (uint16) or e4m3 codes (uint8), row-major, d_h fastest.  A "row"
 * is the flat index (b * n_q + h) * Lq + i of one query.
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

int oracle_version(void) { return 4; }

/* A bf16 bit pattern is the upper half of an fp32 bit pattern, so widening is
 * exact: shift into place, reinterpret as float, convert to double. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* An OCP e4m3 code, decoded from the format's definition: sign bit 7,
 * exponent bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 holds the
 * subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN (there is no
 * infinity).  Exact in double. */
static double widen_e4m3(uint8_t code)
{
    const int sign = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    double x;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        x = ldexp((double)m, -9);
    else
        x = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -x : x;
}

enum { KIND_BF16 = 0, KIND_E4M3 = 1 };

/* Element idx of a tensor of the given kind, widened exactly, times mul. */
static inline double elem(int kind, const void *base, int64_t idx, double mul)
{
    if (kind == KIND_BF16)
        return widen_bf16(((const uint16_t *)base)[idx]) * mul;
    return widen_e4m3(((const uint8_t *)base)[idx]) * mul;
}

/* One query row, done the plain way.  s and w are scratch rows of length Lk.
 * dq, dk, dv multiply the decoded q, k, v (1 for bf16). */
static void one_row(int kind, const void *q, const void *k, const void *v,
                    int64_t Lq, int64_t Lk, int64_t q_off, int64_t n_q,
                    int64_t n_kv, int64_t d_h, double scale, double dq, double dk,
                    double dv, int causal, int64_t row, double *s, double *w,
                    double *out, double *lse, uint64_t *flops)
{
    const int64_t L = Lk;
    const int64_t g = n_q / n_kv;
    const int64_t i = row % Lq;
    const int64_t h = (row / Lq) % n_q;
    const int64_t b = row / (Lq * n_q);
    const int64_t kvh = h / g;
    const int64_t qrow = ((b * n_q + h) * Lq + i) * d_h;
    const int64_t kbase = (b * n_kv + kvh) * Lk * d_h;
    const int64_t vbase = (b * n_kv + kvh) * Lk * d_h;
    /* visible keys: j <= q_off + i when causal, all Lk keys otherwise */
    const int64_t n_vis = causal ? q_off + i + 1 : Lk;

    /* 1. materialise the whole score row; masked entries are -inf and their
     *    dot products are never formed */
    for (int64_t j = 0; j < L; ++j) {
        if (j < n_vis) {
            const int64_t krow = kbase + j * d_h;
            double dot = 0.0;
            for (int64_t t = 0; t < d_h; ++t)
                dot += elem(kind, q, qrow + t, dq) * elem(kind, k, krow + t, dk);
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
        const int64_t vrow = vbase + j * d_h;
        const double p = w[j];
        for (int64_t t = 0; t < d_h; ++t)
            out[t] += p * elem(kind, v, vrow + t, dv);
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
static int rows_generic(int kind, const void *q, const void *k, const void *v,
                        int64_t B, int64_t Lq, int64_t Lk, int64_t q_off,
                        int64_t n_q, int64_t n_kv, int64_t d_h, float scale,
                        double dq, double dk, double dv,
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
            one_row(kind, q, k, v, Lq, Lk, q_off, n_q, n_kv, d_h, sc, dq, dk, dv, causal,
                    row, s, w, out + r * d_h, lse + r, &count);
        }
        free(s);
        free(w);
    }
    *flops = count;
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

int oracle_attn_rows_chunk(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                           int64_t B, int64_t Lq, int64_t Lk, int64_t q_off,
                           int64_t n_q, int64_t n_kv, int64_t d_h, float scale,
                           int causal, const int64_t *rows, int64_t n_rows,
                           double *out, double *lse, uint64_t *flops, int threads)
{
    return rows_generic(KIND_BF16, q, k, v, B, Lq, Lk, q_off, n_q, n_kv, d_h, scale,
                        1.0, 1.0, 1.0, causal, rows, n_rows, out, lse, flops, threads);
}

/*
 * The chunk with e4m3 inputs: q, k, v are OCP e4m3 codes, decoded exactly
 * and multiplied by descale_q, descale_k, descale_v (fp32 values, widened
 * exactly).  Arguments and results otherwise as oracle_attn_rows_chunk.
 */
int oracle_attn_rows_chunk_fp8(const uint8_t *q, const uint8_t *k, const uint8_t *v,
                               int64_t B, int64_t Lq, int64_t Lk, int64_t q_off,
                               int64_t n_q, int64_t n_kv, int64_t d_h, float scale,
                               float descale_q, float descale_k, float descale_v,
                               int causal, const int64_t *rows, int64_t n_rows,
                               double *out, double *lse, uint64_t *flops, int threads)
{
    if (!isfinite(descale_q) || !isfinite(descale_k) || !isfinite(descale_v))
        return ORACLE_BAD_ARG;
    return rows_generic(KIND_E4M3, q, k, v, B, Lq, Lk, q_off, n_q, n_kv, d_h, scale,
                        (double)descale_q, (double)descale_k, (double)descale_v, causal,
                        rows, n_rows, out, lse, flops, threads);
}

/* Decoded value of every e4m3 code (for pinning the decoder): out[256]. */
void oracle_e4m3_table(double *out)
{
    for (int c = 0; c < 256; ++c)
        out[c] = widen_e4m3((uint8_t)c);
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

/* ------------------------------------------------------------------------
 * Backward pass: the gradients of the attention output with respect to Q, K
 * and V for an upstream gradient dO, recomputed from the saved row
 * statistic ("Long-Context Attention Explained", section "What
 * FlashAttention does not change": the backward pass needs the small saved
 * row statistics, not the score matrix).  Written out from the definition
 * O_i = sum_j P_ij v_j, P_ij = exp(s_ij - LSE_i), s_ij = scale q_i . k_j:
 *     dV_j  = sum_i P_ij dO_i                      (over the query heads of
 *     dP_ij = dO_i . v_j                             the group and the rows
 *     D_i   = sum_j P_ij dP_ij  (= dO_i . O_i)        that see key j)
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dQ_i  = scale sum_j dS_ij k_j
 *     dK_j  = scale sum_i dS_ij q_i
 * Whole sequences only (Lq = Lk = L, query i sees j <= i when causal).
 * ------------------------------------------------------------------------ */

/* Per-row statistics for the backward pass, for the requested query rows
 * (flat (b * n_q + h) * L + i; rows == NULL: every row, n_rows = B n_q L):
 * lse[r] (natural log, as the forward oracle) and delta[r] = sum_t dO[r,t]
 * O[r,t] with O the exact output, in fp64; out (NULL or [n_rows, d_h])
 * receives that output. */
int oracle_attn_bwd_rowstats(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                             const uint16_t *dout, int64_t B, int64_t L, int64_t n_q,
                             int64_t n_kv, int64_t d_h, float scale, int causal,
                             const int64_t *rows, int64_t n_rows, double *out, double *lse,
                             double *delta, int threads)
{
    if (!dout || !delta) return ORACLE_BAD_ARG;
    double *o = out;
    if (!o) {
        o = (double *)malloc((size_t)n_rows * (size_t)d_h * sizeof(double));
        if (!o) return ORACLE_NO_MEMORY;
    }
    uint64_t flops = 0;
    int rc = rows_generic(KIND_BF16, q, k, v, B, L, L, 0, n_q, n_kv, d_h, scale, 1.0, 1.0, 1.0,
                          causal, rows, n_rows, o, lse, &flops, threads);
    if (rc == ORACLE_OK) {
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t row = rows ? rows[r] : r;
            double acc = 0.0;
            for (int64_t t = 0; t < d_h; ++t)
                acc += widen_bf16(dout[row * d_h + t]) * o[r * d_h + t];
            delta[r] = acc;
        }
    }
    if (o != out) free(o);
    return rc;
}

/* Weight P_ij of query row (b, h, i) on key j of its kv head, from the
 * exact row statistic lse_i; 0 for a masked key. */
static double bwd_weight(const uint16_t *q, const uint16_t *k, int64_t L, int64_t n_q,
                         int64_t n_kv, int64_t d_h, double scale, int causal, int64_t b,
                         int64_t h, int64_t i, int64_t j, double lse_i)
{
    if (causal && j > i) return 0.0;
    const int64_t kvh = h / (n_q / n_kv);
    const uint16_t *qrow = q + ((b * n_q + h) * L + i) * d_h;
    const uint16_t *krow = k + ((b * n_kv + kvh) * L + j) * d_h;
    double dot = 0.0;
    for (int64_t t = 0; t < d_h; ++t)
        dot += widen_bf16(qrow[t]) * widen_bf16(krow[t]);
    return exp(scale * dot - lse_i);
}

/* dP_ij = dO_i . v_j */
static double bwd_dp(const uint16_t *v, const uint16_t *dout, int64_t L, int64_t n_q,
                     int64_t n_kv, int64_t d_h, int64_t b, int64_t h, int64_t i, int64_t j)
{
    const int64_t kvh = h / (n_q / n_kv);
    const uint16_t *drow = dout + ((b * n_q + h) * L + i) * d_h;
    const uint16_t *vrow = v + ((b * n_kv + kvh) * L + j) * d_h;
    double acc = 0.0;
    for (int64_t t = 0; t < d_h; ++t)
        acc += widen_bf16(drow[t]) * widen_bf16(vrow[t]);
    return acc;
}

/* dQ for the requested query rows (flat (b * n_q + h) * L + i):
 * dq [n_rows, d_h] fp64.  lse and delta: every row's statistics (indexed by
 * flat row; only the requested rows' entries are read). */
int oracle_attn_bwd_dq(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const uint16_t *dout, int64_t B, int64_t L, int64_t n_q, int64_t n_kv,
                       int64_t d_h, float scale, int causal, const double *lse,
                       const double *delta, const int64_t *rows, int64_t n_rows, double *dq,
                       int threads)
{
    if (!q || !k || !v || !dout || !lse || !delta || !rows || !dq) return ORACLE_BAD_ARG;
    if (B < 1 || L < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || n_q % n_kv) return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * n_q * L) return ORACLE_BAD_ARG;
    const double sc = (double)scale;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t row = rows[r];
        const int64_t i = row % L, h = (row / L) % n_q, b = row / (L * n_q);
        const int64_t kvh = h / (n_q / n_kv);
        double *out = dq + r * d_h;
        for (int64_t t = 0; t < d_h; ++t) out[t] = 0.0;
        const int64_t n_vis = causal ? i + 1 : L;
        for (int64_t j = 0; j < n_vis; ++j) {
            const double p = bwd_weight(q, k, L, n_q, n_kv, d_h, sc, causal, b, h, i, j, lse[row]);
            const double ds = p * (bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j) - delta[row]);
            const uint16_t *krow = k + ((b * n_kv + kvh) * L + j) * d_h;
            for (int64_t t = 0; t < d_h; ++t) out[t] += sc * ds * widen_bf16(krow[t]);
        }
    }
    return ORACLE_OK;
}

/* dK and dV for the requested key rows (flat (b * n_kv + kvh) * L + j):
 * dk, dv [n_rows, d_h] fp64, summed over the g query heads of the group and
 * every query row that sees key j.  lse and delta as for oracle_attn_bwd_dq;
 * the entries of the query rows that see a requested key are read. */
int oracle_attn_bwd_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                         const uint16_t *dout, int64_t B, int64_t L, int64_t n_q, int64_t n_kv,
                         int64_t d_h, float scale, int causal, const double *lse,
                         const double *delta, const int64_t *rows, int64_t n_rows, double *dk,
                         double *dv, int threads)
{
    if (!q || !k || !v || !dout || !lse || !delta || !rows || !dk || !dv) return ORACLE_BAD_ARG;
    if (B < 1 || L < 1 || n_q < 1 || n_kv < 1 || d_h < 1 || n_q % n_kv) return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n_rows; ++r)
        if (rows[r] < 0 || rows[r] >= B * n_kv * L) return ORACLE_BAD_ARG;
    const double sc = (double)scale;
    const int64_t g = n_q / n_kv;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        const int64_t row = rows[r];
        const int64_t j = row % L, kvh = (row / L) % n_kv, b = row / (L * n_kv);
        double *ok = dk + r * d_h, *ov = dv + r * d_h;
        for (int64_t t = 0; t < d_h; ++t) ok[t] = ov[t] = 0.0;
        for (int64_t h = kvh * g; h < kvh * g + g; ++h) {
            for (int64_t i = causal ? j : 0; i < L; ++i) {
                const int64_t qrow_id = (b * n_q + h) * L + i;
                const double p = bwd_weight(q, k, L, n_q, n_kv, d_h, sc, causal, b, h, i, j,
                                            lse[qrow_id]);
                const double ds =
                    p * (bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j) - delta[qrow_id]);
                const uint16_t *qrow = q + qrow_id * d_h;
                const uint16_t *drow = dout + qrow_id * d_h;
                for (int64_t t = 0; t < d_h; ++t) {
                    ov[t] += p * widen_bf16(drow[t]);
                    ok[t] += sc * ds * widen_bf16(qrow[t]);
                }
            }
        }
    }
    return ORACLE_OK;
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
