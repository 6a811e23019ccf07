/*
 * gdn_scan_ref.c -- CPU oracle: the gated delta rule, one token at a time, in
 * IEEE double precision.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no source, header, table or
 * helper with the HIP library; neither side includes or links the other.
 *
 * What it computes (LT2: Linear-Time Looped Transformers, Section 2 "LT2"
 * paragraph: q_t, k_t in R^{dk}, v_t in R^{dv} are per-token projections and
 * S_t in R^{dk x dv} is the recurrent state of the linear-attention mixer; the
 * mixer is Gated DeltaNet, Appendix C; Appendix B.1 describes one block as a
 * diagonal-plus-low-rank, rank-1 state update; Fig. 6 caption: data-dependent
 * gating plus the delta rule).  The update the pages name but do not print is
 * read as the gated delta rule of "Gated delta networks: Improving mamba2 with
 * delta rule" (reference [70] of the LT2 pages):
 *
 *     S_t = alpha_t * (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t                      (post-update state, no 1/sqrt(dk))
 *
 * Elementwise, with (k^T S)_j = sum_i k_i S_ij:
 *     S_ij <- alpha * (S_ij - beta * k_i * (k^T S)_j) + beta * k_i * v_j
 *     o_j   = sum_i q_i S_ij
 *
 * Layouts (row-major, last index fastest):
 *     q, k   [B, L, H, dk]      v, o  [B, L, H, dv]
 *     alpha, beta [B, L, H]     s_init, s_final [B, H, dk, dv]
 * s_init == NULL starts every (b, h) from S = 0.  s_final may be NULL.
 * s_final may alias s_init (the state is copied before the scan starts).
 */
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, -1 if scratch memory could not be allocated. */
int oracle_scan(int B, int L, int H, int dk, int dv,
                const double *q, const double *k, const double *v,
                const double *alpha, const double *beta,
                const double *s_init, double *o, double *s_final)
{
    int failed = 0;
    long pairs = (long)B * H;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: failed)
    for (long p = 0; p < pairs; ++p) {
        int b = (int)(p / H), h = (int)(p % H);
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *kS = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !kS) { free(S); free(kS); failed = 1; continue; }
        if (s_init)
            memcpy(S, s_init + (size_t)p * dk * dv, sizeof(double) * (size_t)dk * dv);
        else
            memset(S, 0, sizeof(double) * (size_t)dk * dv);

        for (int t = 0; t < L; ++t) {
            size_t row = ((size_t)b * L + t) * H + h;
            const double *qt = q + row * dk;
            const double *kt = k + row * dk;
            const double *vt = v + row * dv;
            double a = alpha[row], be = beta[row];
            double *ot = o + row * dv;

            /* (k_t^T S_{t-1})_j */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += kt[i] * S[(size_t)i * dv + j];
                kS[j] = acc;
            }
            /* S_t = alpha (S - beta k (k^T S)) + beta k v^T */
            for (int i = 0; i < dk; ++i)
                for (int j = 0; j < dv; ++j) {
                    double s = S[(size_t)i * dv + j];
                    S[(size_t)i * dv + j] = a * (s - be * kt[i] * kS[j]) + be * kt[i] * vt[j];
                }
            /* o_t = S_t^T q_t */
            for (int j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int i = 0; i < dk; ++i) acc += qt[i] * S[(size_t)i * dv + j];
                ot[j] = acc;
            }
        }
        if (s_final)
            memcpy(s_final + (size_t)p * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(kS);
    }
    return failed ? -1 : 0;
}
