/*
 * la_oracle.c -- CPU reference ("oracle") for causal linear attention as used
 * by Lightning Attention.  TEST INFRASTRUCTURE ONLY: the product library never
 * links, loads or calls this file; only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark do.
 *
 * Everything is computed in IEEE double with plain loops, one sequence (unit)
 * at a time, no blocking beyond what the method itself defines.  Inputs arrive
 * as float (bf16 and fp32 inputs are both exactly representable in float) and
 * are widened to double losslessly before any arithmetic.
 *
 * Sources (the pages these functions follow):
 *   [W]  wiki page "MiniMax-01 Lightning Attention", section "Lightning
 *        Attention 设计" (intra-block left product, inter-block right product
 *        with a recursively updated KV state, O(nd^2 + nBd) cost, O(d^2)
 *        per-token inference) and the comparison table in section
 *        "与标准 Softmax Attention 的区别" (a d x d KV state replaces the KV
 *        cache).
 *   [T]  Tencent Cloud article "首个线性注意力架构的大模型来了…", section 4.1
 *        (blocks of e.g. 256 tokens; each block attends inside itself, and all
 *        earlier blocks are compressed into one compact key-value prefix).
 *
 * The operation is causal linear attention with identity feature map, no
 * normaliser and no decay: o_i = sum_{j<=i} (q_i . k_j) v_j.  No scale is
 * applied inside the operation.
 *
 * Layouts (all row-major): a unit is one (sequence, head) stream of n tokens;
 * q, k, v are [n][d]; o is [n][d]; a state S is [d][d] with S[a][b] =
 * sum_t k_t[a] v_t[b] (row = key dimension, column = value dimension).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC (no fast-math).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- single-unit forms ------------------------------------------------- */

/* Quadratic form, straight from the definition of causal linear attention
 * ([W] "Lightning Attention 设计": linear attention with a causal mask).
 * o_i = sum_{j=0..i} (sum_a q_i[a] k_j[a]) * v_j.   O(n^2 d). */
void lao_naive(const float *q, const float *k, const float *v, double *o,
               int64_t n, int d)
{
    for (int64_t i = 0; i < n; ++i) {
        double *oi = o + i * d;
        for (int b = 0; b < d; ++b) oi[b] = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int a = 0; a < d; ++a)
                s += (double)q[i * d + a] * (double)k[j * d + a];
            for (int b = 0; b < d; ++b)
                oi[b] += s * (double)v[j * d + b];
        }
    }
}

/* Token-by-token recurrent form ([W] "Lightning Attention 设计": inference
 * only updates the KV state, O(d^2) per token; [T] 4.1: generation keeps
 * updating the prefix).  Inclusive: token t sees itself.
 *   S <- S + k_t^T v_t ;  o_t = q_t S .
 * S_io (d*d doubles) holds the initial state on entry (NULL = zero) and the
 * final state on exit when non-NULL.  O(n d^2). */
void lao_recurrent(const float *q, const float *k, const float *v, double *o,
                   int64_t n, int d, double *S_io)
{
    double *S = S_io ? S_io : (double *)calloc((size_t)d * d, sizeof(double));
    for (int64_t t = 0; t < n; ++t) {
        const float *kt = k + t * d, *vt = v + t * d, *qt = q + t * d;
        for (int a = 0; a < d; ++a) {
            double ka = (double)kt[a];
            double *Sa = S + (size_t)a * d;
            for (int b = 0; b < d; ++b) Sa[b] += ka * (double)vt[b];
        }
        double *ot = o + t * d;
        for (int b = 0; b < d; ++b) ot[b] = 0.0;
        for (int a = 0; a < d; ++a) {
            double qa = (double)qt[a];
            const double *Sa = S + (size_t)a * d;
            for (int b = 0; b < d; ++b) ot[b] += qa * Sa[b];
        }
    }
    if (!S_io) free(S);
}

/* Recurrent form that only emits o at the requested token positions
 * (rows[] strictly increasing, each in [0, n)).  Same arithmetic as
 * lao_recurrent for the state; used to check sampled outputs of very long
 * sequences without storing all of o. */
void lao_recurrent_rows(const float *q, const float *k, const float *v,
                        int64_t n, int d, const int64_t *rows, int64_t nrows,
                        double *o_rows)
{
    double *S = (double *)calloc((size_t)d * d, sizeof(double));
    int64_t r = 0;
    for (int64_t t = 0; t < n && r < nrows; ++t) {
        const float *kt = k + t * d, *vt = v + t * d;
        for (int a = 0; a < d; ++a) {
            double ka = (double)kt[a];
            double *Sa = S + (size_t)a * d;
            for (int b = 0; b < d; ++b) Sa[b] += ka * (double)vt[b];
        }
        if (rows[r] == t) {
            const float *qt = q + t * d;
            double *ot = o_rows + r * d;
            for (int b = 0; b < d; ++b) ot[b] = 0.0;
            for (int a = 0; a < d; ++a) {
                double qa = (double)qt[a];
                const double *Sa = S + (size_t)a * d;
                for (int b = 0; b < d; ++b) ot[b] += qa * Sa[b];
            }
            ++r;
        }
    }
    free(S);
}

/* Block form with block size B, in the order the pages describe it ([W]
 * "Lightning Attention 设计"; [T] 4.1): for each block of B tokens,
 *   intra (left product):  P = Q_b K_b^T with entries j > i set to 0, then P V_b
 *   inter (right product): Q_b S, with S the sum of k^T v over all EARLIER
 *                          blocks (the compact key-value prefix)
 *   o_b = intra + inter ; then S <- S + K_b^T V_b.
 * Blocks start at token 0; the last one may be short.  It is mathematically
 * identical to lao_naive for every B >= 1 (up to rounding order). */
void lao_block(const float *q, const float *k, const float *v, double *o,
               int64_t n, int d, int64_t B)
{
    double *S = (double *)calloc((size_t)d * d, sizeof(double));
    double *P = (double *)malloc((size_t)B * B * sizeof(double));
    for (int64_t s0 = 0; s0 < n; s0 += B) {
        int64_t nb = (n - s0 < B) ? (n - s0) : B;
        const float *Qb = q + s0 * d, *Kb = k + s0 * d, *Vb = v + s0 * d;
        double *Ob = o + s0 * d;
        /* P = mask(Q_b K_b^T) */
        for (int64_t i = 0; i < nb; ++i)
            for (int64_t j = 0; j < nb; ++j) {
                double s = 0.0;
                if (j <= i)
                    for (int a = 0; a < d; ++a)
                        s += (double)Qb[i * d + a] * (double)Kb[j * d + a];
                P[i * B + j] = s;
            }
        for (int64_t i = 0; i < nb; ++i) {
            double *oi = Ob + i * d;
            /* left product P V_b */
            for (int b = 0; b < d; ++b) {
                double acc = 0.0;
                for (int64_t j = 0; j < nb; ++j) acc += P[i * B + j] * (double)Vb[j * d + b];
                oi[b] = acc;
            }
            /* right product Q_b S (S = prefix of earlier blocks) */
            for (int b = 0; b < d; ++b) {
                double acc = 0.0;
                for (int a = 0; a < d; ++a) acc += (double)Qb[i * d + a] * S[(size_t)a * d + b];
                oi[b] += acc;
            }
        }
        /* S <- S + K_b^T V_b */
        for (int a = 0; a < d; ++a)
            for (int b = 0; b < d; ++b) {
                double acc = 0.0;
                for (int64_t j = 0; j < nb; ++j) acc += (double)Kb[j * d + a] * (double)Vb[j * d + b];
                S[(size_t)a * d + b] += acc;
            }
    }
    free(P);
    free(S);
}

/* One decode step in the literal order of the decode recurrence: the output
 * reads the state BEFORE this token's update, then the state absorbs the token.
 *   o = q S_old ;  S_new = S_old + k^T v .
 * ([W] "Lightning Attention 设计": O(d^2) per token, independent of length;
 * table row "状态大小": a d x d KV state.) */
void lao_decode_step(const float *q, const float *k, const float *v,
                     double *S, double *o, int d)
{
    for (int b = 0; b < d; ++b) {
        double acc = 0.0;
        for (int a = 0; a < d; ++a) acc += (double)q[a] * S[(size_t)a * d + b];
        o[b] = acc;
    }
    for (int a = 0; a < d; ++a) {
        double ka = (double)k[a];
        for (int b = 0; b < d; ++b) S[(size_t)a * d + b] += ka * (double)v[b];
    }
}

/* ---- batched drivers (parallel over independent units only) ----------- */

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

int lao_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* units independent [n][d] streams laid out back to back ([units][n][d]).
 * form: 0 = naive, 1 = recurrent, 2 = block (block_size B). */
void lao_units(const float *q, const float *k, const float *v, double *o,
               int64_t units, int64_t n, int d, int form, int64_t B,
               int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        size_t off = (size_t)u * (size_t)n * (size_t)d;
        if (form == 0)      lao_naive(q + off, k + off, v + off, o + off, n, d);
        else if (form == 1) lao_recurrent(q + off, k + off, v + off, o + off, n, d, NULL);
        else                lao_block(q + off, k + off, v + off, o + off, n, d, B);
    }
}

/* Packed variable-length input: tensors [heads][T][d], sequence s occupies
 * tokens [cu[s], cu[s+1]) of every head and starts from an empty state.
 * form as in lao_units. */
void lao_varlen(const float *q, const float *k, const float *v, double *o,
                int heads, int64_t T, const int32_t *cu, int nseq, int d,
                int form, int64_t B, int nthreads)
{
    set_threads(nthreads);
    int64_t total = (int64_t)heads * nseq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < total; ++x) {
        int h = (int)(x / nseq), s = (int)(x % nseq);
        int64_t n = (int64_t)cu[s + 1] - cu[s];
        size_t off = ((size_t)h * (size_t)T + (size_t)cu[s]) * (size_t)d;
        if (n <= 0) continue;
        if (form == 0)      lao_naive(q + off, k + off, v + off, o + off, n, d);
        else if (form == 1) lao_recurrent(q + off, k + off, v + off, o + off, n, d, NULL);
        else                lao_block(q + off, k + off, v + off, o + off, n, d, B);
    }
}

/* Recurrent form over `units` independent [n][d] streams ([units][n][d]),
 * each starting from its own state: S0 [units][d][d] (NULL = zero) and
 * ending with its final state written to Sf [units][d][d] (NULL = not
 * wanted).  o_t = q_t (S0 + sum_{j<=t} k_j^T v_j), S_final = S0 + sum k^T v.
 * This is the state a prefill hands to decoding, or to the next piece of a
 * sequence prefilled in pieces ([W] "Lightning Attention 设计": the KV state
 * carries everything earlier tokens contribute). */
void lao_units_state(const float *q, const float *k, const float *v, double *o,
                     int64_t units, int64_t n, int d, const double *S0, double *Sf,
                     int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        size_t off = (size_t)u * (size_t)n * (size_t)d, dd = (size_t)d * d;
        double *S = (double *)malloc(dd * sizeof(double));
        for (size_t e = 0; e < dd; ++e) S[e] = S0 ? S0[(size_t)u * dd + e] : 0.0;
        lao_recurrent(q + off, k + off, v + off, o + off, n, d, S);
        if (Sf)
            for (size_t e = 0; e < dd; ++e) Sf[(size_t)u * dd + e] = S[e];
        free(S);
    }
}

/* Packed input as in lao_varlen, recurrent form, with per-sequence states
 * S0 / Sf laid out [nseq][heads][d][d] (NULL as in lao_units_state).  A
 * sequence of length 0 ends in its initial state. */
void lao_varlen_state(const float *q, const float *k, const float *v, double *o,
                      int heads, int64_t T, const int32_t *cu, int nseq, int d,
                      const double *S0, double *Sf, int nthreads)
{
    set_threads(nthreads);
    int64_t total = (int64_t)heads * nseq;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t x = 0; x < total; ++x) {
        int h = (int)(x / nseq), s = (int)(x % nseq);
        int64_t n = (int64_t)cu[s + 1] - cu[s];
        size_t off = ((size_t)h * (size_t)T + (size_t)cu[s]) * (size_t)d, dd = (size_t)d * d;
        size_t so = ((size_t)s * heads + h) * dd;
        double *S = (double *)malloc(dd * sizeof(double));
        for (size_t e = 0; e < dd; ++e) S[e] = S0 ? S0[so + e] : 0.0;
        if (n > 0) lao_recurrent(q + off, k + off, v + off, o + off, n, d, S);
        if (Sf)
            for (size_t e = 0; e < dd; ++e) Sf[so + e] = S[e];
        free(S);
    }
}

/* `steps` decode steps over `units` independent states.
 * q, k, v: [steps][units][d]; S: [units][d][d] (in/out); o: [steps][units][d]. */
void lao_decode_units(const float *q, const float *k, const float *v,
                      double *S, double *o, int64_t steps, int64_t units,
                      int d, int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < units; ++u) {
        double *Su = S + (size_t)u * d * d;
        for (int64_t t = 0; t < steps; ++t) {
            size_t off = ((size_t)t * (size_t)units + (size_t)u) * (size_t)d;
            lao_decode_step(q + off, k + off, v + off, Su, o + off, d);
        }
    }
}
