/*
 * gdr_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU model of the gated delta rule, used to check the
 * HIP library.  It is called only by the tests, by the smoke check and by the
 * benchmark's CPU-baseline leg; the library never links or calls it.  It
 * shares no code with the HIP path.
 *
 * What it computes is the per-token recurrence of the Qwen3-Next blog post
 * ("Code-Qwen3-Next", section 5(2), the token-by-token rule), written in the
 * value-by-key orientation of the state (S[i][j]: i = value index, j = key
 * index, as in the Ascend operator page's state_new [Dv, Dk]):
 *
 *   for each sequence b and value head h (query/key head j = h / (Nv / Nqk)):
 *     S = state_in[b][h]            (zeros when no initial state is given)
 *     for each token t of the sequence, in order:
 *       kh = k[t][j] / sqrt(|k[t][j]|^2 + eps)
 *       qh = scale * q[t][j] / sqrt(|q[t][j]|^2 + eps)
 *       S  = exp(g[t][h]) * S                      (decay first ...)
 *       u  = S kh                                  (... then read)
 *       S  = S + beta[t][h] * (v[t][h] - u) kh^T   (delta-rule write)
 *       out[t][h] = S qh                           (read after the write)
 *     state_out[b][h] = S
 *
 * The L2 normalisation x / sqrt(sum x^2 + eps) is the Ascend operator page's
 * formula (section "math formulas"); eps = 1e-6 in every caller.  With
 * l2norm = 0 the normalisation is skipped (kh = k, qh = scale * q), the
 * blog's use_qk_l2norm_in_kernel = False.  Rows of S
 * evolve independently of each other (every step acts on each row alone), so
 * the work is split over (sequence, head, block of rows) with OpenMP.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ROWS_PER_TASK 16

/* Returns 0 on success, a negative number for invalid arguments. */
int gdr_oracle_run(const double* q, const double* k, const double* v,
                   const double* g, const double* beta,
                   const double* state_in,      /* [N][Nv][Dv][Dk] or NULL */
                   const int32_t* cu_seqlens,   /* [N+1] */
                   int32_t N, int32_t Nqk, int32_t Nv, int32_t Dk, int32_t Dv,
                   double scale, double eps, int32_t l2norm,
                   double* out,                 /* [T][Nv][Dv] */
                   double* state_out,           /* [N][Nv][Dv][Dk] or NULL */
                   int32_t nthreads)
{
    if (N < 0 || Nqk <= 0 || Nv <= 0 || Dk <= 0 || Dv <= 0) return -1;
    if (Nv % Nqk != 0) return -2;
    if (cu_seqlens[0] != 0) return -3;
    for (int32_t b = 0; b < N; ++b)
        if (cu_seqlens[b + 1] < cu_seqlens[b]) return -3;
    const int32_t group = Nv / Nqk;
    const int32_t row_blocks = (Dv + ORACLE_ROWS_PER_TASK - 1) / ORACLE_ROWS_PER_TASK;
    const int64_t tasks = (int64_t)N * Nv * row_blocks;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double* S = (double*)malloc(sizeof(double) * (size_t)ORACLE_ROWS_PER_TASK * (size_t)Dk);
        double* kh = (double*)malloc(sizeof(double) * (size_t)Dk);
        double* qh = (double*)malloc(sizeof(double) * (size_t)Dk);

#pragma omp for schedule(dynamic, 1)
        for (int64_t task = 0; task < tasks; ++task) {
            const int32_t rb = (int32_t)(task % row_blocks);
            const int32_t h = (int32_t)((task / row_blocks) % Nv);
            const int32_t b = (int32_t)(task / ((int64_t)row_blocks * Nv));
            const int32_t j = h / group;
            const int32_t r0 = rb * ORACLE_ROWS_PER_TASK;
            const int32_t r1 = (r0 + ORACLE_ROWS_PER_TASK < Dv) ? r0 + ORACLE_ROWS_PER_TASK : Dv;
            const int32_t nr = r1 - r0;
            const size_t state_off = ((size_t)b * Nv + h) * (size_t)Dv * Dk;

            /* initial state rows */
            for (int32_t r = 0; r < nr; ++r)
                for (int32_t c = 0; c < Dk; ++c)
                    S[(size_t)r * Dk + c] =
                        state_in ? state_in[state_off + (size_t)(r0 + r) * Dk + c] : 0.0;

            for (int32_t t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
                const double* kt = k + ((size_t)t * Nqk + j) * Dk;
                const double* qt = q + ((size_t)t * Nqk + j) * Dk;
                double ssk = 0.0, ssq = 0.0;
                for (int32_t c = 0; c < Dk; ++c) { ssk += kt[c] * kt[c]; ssq += qt[c] * qt[c]; }
                const double rk = l2norm ? 1.0 / sqrt(ssk + eps) : 1.0;
                const double rq = l2norm ? scale / sqrt(ssq + eps) : scale;
                for (int32_t c = 0; c < Dk; ++c) { kh[c] = kt[c] * rk; qh[c] = qt[c] * rq; }
                const double alpha = exp(g[(size_t)t * Nv + h]);
                const double bt = beta[(size_t)t * Nv + h];
                const double* vt = v + ((size_t)t * Nv + h) * Dv;
                double* ot = out + ((size_t)t * Nv + h) * Dv;

                for (int32_t r = 0; r < nr; ++r) {
                    double* Sr = S + (size_t)r * Dk;
                    double u = 0.0;
                    for (int32_t c = 0; c < Dk; ++c) { Sr[c] *= alpha; u += Sr[c] * kh[c]; }
                    const double delta = bt * (vt[r0 + r] - u);
                    double o = 0.0;
                    for (int32_t c = 0; c < Dk; ++c) { Sr[c] += delta * kh[c]; o += Sr[c] * qh[c]; }
                    ot[r0 + r] = o;
                }
            }
            if (state_out)
                for (int32_t r = 0; r < nr; ++r)
                    for (int32_t c = 0; c < Dk; ++c)
                        state_out[state_off + (size_t)(r0 + r) * Dk + c] = S[(size_t)r * Dk + c];
        }
        free(S); free(kh); free(qh);
    }
    return 0;
}

/* Number of threads an OpenMP parallel region would use after a request. */
int gdr_oracle_threads(int32_t nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int n = 0;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
#else
    (void)nthreads;
    return 1;
#endif
}
