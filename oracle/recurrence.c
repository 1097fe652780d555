/*
 * oracle/recurrence.c -- the per-token recurrent form of linear attention,
 * in fp64, one (request, head) tile at a time.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP kernels are
 * checked against.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load it.  It shares no code, header or constant
 * with the GPU library.
 *
 * What it computes (KVBuffer: IO-aware Serving for Linear Attention, pith.science
 * page, abstract: the serving systems it improves on read and rewrite the
 * whole state for every decoded token; Figure 3 caption: that recurrent form
 * is the buffer-size-0 case).  The pages give no
 * equation; the three update rules below are the ones the workload definitions
 * fix, each applied once per token t with S the d_k x d_v state:
 *
 *   rule 0, ungated linear attention:  S_t = S_{t-1} + k_t v_t^T
 *   rule 1, scalar-gated:              S_t = exp(g_t) S_{t-1} + k_t v_t^T
 *   rule 2, gated delta rule:          S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1}
 *                                            + beta_t k_t v_t^T
 *   rule 3, per-channel gate:          S_t = diag(exp(g_t)) S_{t-1} + k_t v_t^T,
 *                                      g_t a vector over the d_k key channels
 *
 * Rule 3 is the diagonal decay of the gated linear attention and matrix-state
 * RNN families the same page lists among its references ([20] gated linear
 * attention, [13] RWKV with matrix-valued states): row r of the state (key
 * channel r) decays by exp(g_t[r]).
 *
 * and the output of token t is o_t = S_t^T (scale * q_t): the state after the
 * token's own update is the one that is read (the current token attends to
 * itself).
 *
 * For rule 2 the product (I - beta k k^T) S is formed as S - beta k (k^T S):
 * that is the matrix product with the identity-minus-rank-one matrix written
 * out, evaluated without materialising the d_k x d_k matrix.  A test checks it
 * against the explicit matrix product.
 *
 * Layouts (all row-major, fp64):
 *   S     [ntiles][dk][dv]       state in / out
 *   q, k  [nsteps][ntiles][dk]
 *   v     [nsteps][ntiles][dv]
 *   g, beta [nsteps][ntiles]     (g may be NULL for rule 0; beta only for rule 2)
 *   g       [nsteps][ntiles][dk] for rule 3
 *   out   [nsteps][ntiles][dv]
 *   mag   [nsteps][ntiles][dv] or NULL: |S_t|^T |scale q_t|, the output
 *         computed with every term's absolute value -- the size of the
 *         product that defines o_t, against which the error of a result
 *         accumulated in finite precision is measured
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void oracle_one_tile(int rule, long tile, long ntiles, int nsteps, int dk, int dv,
                            double scale, double* S, const double* q, const double* k,
                            const double* v, const double* g, const double* beta,
                            double* out, double* mag, double* work)
{
    for (int t = 0; t < nsteps; ++t) {
        const double* qt = q + ((size_t)t * ntiles + tile) * dk;
        const double* kt = k + ((size_t)t * ntiles + tile) * dk;
        const double* vt = v + ((size_t)t * ntiles + tile) * dv;
        double* ot = out + ((size_t)t * ntiles + tile) * dv;
        double gamma = 1.0;
        if (rule == 1 || rule == 2) gamma = exp(g[(size_t)t * ntiles + tile]);

        if (rule == 2) {
            double b = beta[(size_t)t * ntiles + tile];
            /* work = k^T S  (a row vector of length dv) */
            for (int c = 0; c < dv; ++c) work[c] = 0.0;
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) work[c] += kt[r] * S[(size_t)r * dv + c];
            /* S = gamma (S - beta k (k^T S)) + beta k v^T */
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) {
                    double* s = &S[(size_t)r * dv + c];
                    *s = gamma * (*s - b * kt[r] * work[c]) + b * kt[r] * vt[c];
                }
        } else if (rule == 3) {
            /* S = diag(exp(g_t)) S + k v^T: row r decays with its own gate */
            const double* gt = g + ((size_t)t * ntiles + tile) * dk;
            for (int r = 0; r < dk; ++r) {
                const double gr = exp(gt[r]);
                for (int c = 0; c < dv; ++c) {
                    double* s = &S[(size_t)r * dv + c];
                    *s = gr * *s + kt[r] * vt[c];
                }
            }
        } else {
            /* S = gamma S + k v^T   (gamma = 1 for rule 0) */
            for (int r = 0; r < dk; ++r)
                for (int c = 0; c < dv; ++c) {
                    double* s = &S[(size_t)r * dv + c];
                    *s = gamma * *s + kt[r] * vt[c];
                }
        }

        /* o_t = S_t^T (scale q_t) */
        for (int c = 0; c < dv; ++c) ot[c] = 0.0;
        for (int r = 0; r < dk; ++r) {
            double qr = scale * qt[r];
            for (int c = 0; c < dv; ++c) ot[c] += S[(size_t)r * dv + c] * qr;
        }
        if (mag) {
            double* mt = mag + ((size_t)t * ntiles + tile) * dv;
            for (int c = 0; c < dv; ++c) mt[c] = 0.0;
            for (int r = 0; r < dk; ++r) {
                double qa = fabs(scale * qt[r]);
                for (int c = 0; c < dv; ++c) mt[c] += fabs(S[(size_t)r * dv + c]) * qa;
            }
        }
    }
}

/* Runs nsteps tokens of the recurrence on every tile.  Tiles are independent,
 * so with nthreads > 1 they are spread over OpenMP threads (the arithmetic of
 * each tile is unchanged).  Returns 0, or -1 on a bad argument. */
int oracle_recurrent(int rule, long ntiles, int nsteps, int dk, int dv, double scale,
                     double* S, const double* q, const double* k, const double* v,
                     const double* g, const double* beta, double* out, double* mag,
                     int nthreads)
{
    if (rule < 0 || rule > 3 || ntiles < 0 || nsteps < 0 || dk <= 0 || dv <= 0) return -1;
    if (!S || !q || !k || !v || !out) return -1;
    if (rule >= 1 && !g) return -1;
    if (rule == 2 && !beta) return -1;
    if (nthreads < 1) nthreads = 1;
    int bad = 0;
#pragma omp parallel num_threads(nthreads) reduction(| : bad)
    {
        double* work = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!work) bad = 1;
#pragma omp for schedule(static)
        for (long tile = 0; tile < ntiles; ++tile) {
            if (!work) continue;
            oracle_one_tile(rule, tile, ntiles, nsteps, dk, dv, scale,
                            S + (size_t)tile * dk * dv, q, k, v, g, beta, out, mag, work);
        }
        free(work);
    }
    return bad ? -1 : 0;
}

/* Number of threads an OpenMP region gets when asked for n (so a caller can
 * report the threads actually used). */
int oracle_threads_used(int n)
{
    int used = 1;
#ifdef _OPENMP
#pragma omp parallel num_threads(n)
    {
#pragma omp single
        used = omp_get_num_threads();
    }
#else
    (void)n;
#endif
    return used;
}
