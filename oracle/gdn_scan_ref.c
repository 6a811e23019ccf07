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

/*
 * Backward of the same scan: gradients of a loss L(o, S_final) given
 * d_o = dL/do [B, L, H, dv] and d_sfinal = dL/dS_final [B, H, dk, dv] (NULL:
 * zero).  Derived by hand from the recurrence written as
 *     a_t = S_{t-1}^T k_t,  u_t = beta_t (v_t - alpha_t a_t),
 *     S_t = alpha_t S_{t-1} + k_t u_t^T,  o_t = S_t^T q_t.
 * With G = dL/dS_t (everything downstream of S_t), walking t = L .. 1:
 *     G     += q_t d_o_t^T                        (o_t reads S_t)
 *     dq_t   = S_t d_o_t
 *     du     = G^T k_t
 *     dk_t   = G u_t - alpha_t beta_t S_{t-1} du  (k_t u_t^T and a_t)
 *     dv_t   = beta_t du
 *     dbeta_t  = du . (v_t - alpha_t a_t)
 *     dalpha_t = sum_ij G_ij S_{t-1,ij} - beta_t du . a_t
 *     G      = alpha_t G - alpha_t beta_t k_t du^T        (= dL/dS_{t-1})
 * and ds_init = G at the end.  S_{t-1} and S_t are recomputed forward from
 * checkpoints kept every CK tokens (plain recomputation, no other change to
 * the arithmetic).  Outputs may be NULL except dq, dk, dv, dalpha, dbeta.
 * Returns 0, or -1 if scratch memory could not be allocated.
 */
int oracle_scan_backward(int B, int L, int H, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *alpha, const double *beta, const double *s_init,
                         const double *d_o, const double *d_sfinal,
                         double *dq, double *dkk, double *dvv, double *dalpha, double *dbeta,
                         double *ds_init)
{
    enum { CK = 64 };
    int failed = 0;
    long pairs = (long)B * H;
    const size_t SZ = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) reduction(|: failed)
    for (long p = 0; p < pairs; ++p) {
        int b = (int)(p / H), h = (int)(p % H);
        int nck = (L + CK - 1) / CK;
        double *ck = (double *)malloc(sizeof(double) * SZ * (size_t)(nck + 1));   /* S at tokens 0, CK, 2CK, .. */
        double *hist = (double *)malloc(sizeof(double) * SZ * (CK + 1));          /* S_{c0} .. S_{c1} of a block */
        double *G = (double *)malloc(sizeof(double) * SZ);
        double *vec = (double *)malloc(sizeof(double) * (size_t)(3 * dv + dk));
        if (!ck || !hist || !G || !vec) { free(ck); free(hist); free(G); free(vec); failed = 1; continue; }
        double *a = vec, *u = vec + dv, *du = vec + 2 * dv;
        double *S = ck;   /* running state during the checkpoint pass */
        if (s_init) memcpy(S, s_init + (size_t)p * SZ, sizeof(double) * SZ);
        else memset(S, 0, sizeof(double) * SZ);

        /* forward pass: one step of the recurrence, from state `from` into `to` */
#define STEP(from, to, t)                                                                   \
        do {                                                                                \
            size_t row_ = ((size_t)b * L + (t)) * H + h;                                    \
            const double *kt_ = k + row_ * dk, *vt_ = v + row_ * dv;                        \
            double al_ = alpha[row_], be_ = beta[row_];                                     \
            for (int j = 0; j < dv; ++j) {                                                  \
                double acc = 0.0;                                                           \
                for (int i = 0; i < dk; ++i) acc += kt_[i] * (from)[(size_t)i * dv + j];    \
                a[j] = acc;                                                                 \
            }                                                                               \
            for (int i = 0; i < dk; ++i)                                                    \
                for (int j = 0; j < dv; ++j) {                                              \
                    double s_ = (from)[(size_t)i * dv + j];                                 \
                    (to)[(size_t)i * dv + j] = al_ * (s_ - be_ * kt_[i] * a[j]) + be_ * kt_[i] * vt_[j]; \
                }                                                                           \
        } while (0)

        for (int c = 0; c < nck; ++c) {
            double *cur = ck + (size_t)c * SZ, *nxt = ck + (size_t)(c + 1) * SZ;
            int t0 = c * CK, t1 = t0 + CK < L ? t0 + CK : L;
            memcpy(hist, cur, sizeof(double) * SZ);
            for (int t = t0; t < t1; ++t) {
                STEP(hist, hist + SZ, t);
                memcpy(hist, hist + SZ, sizeof(double) * SZ);
            }
            memcpy(nxt, hist, sizeof(double) * SZ);
        }
        /* G = dL/dS_L */
        if (d_sfinal) memcpy(G, d_sfinal + (size_t)p * SZ, sizeof(double) * SZ);
        else memset(G, 0, sizeof(double) * SZ);

        for (int c = nck - 1; c >= 0; --c) {
            int t0 = c * CK, t1 = t0 + CK < L ? t0 + CK : L;
            /* hist[m] = S_{t0 + m}: S after token t0 + m - 1 (hist[0] = state at the block start) */
            memcpy(hist, ck + (size_t)c * SZ, sizeof(double) * SZ);
            for (int t = t0; t < t1; ++t) STEP(hist + (size_t)(t - t0) * SZ, hist + (size_t)(t - t0 + 1) * SZ, t);
            for (int t = t1 - 1; t >= t0; --t) {
                const double *Sp = hist + (size_t)(t - t0) * SZ;       /* S_{t-1} */
                const double *St = hist + (size_t)(t - t0 + 1) * SZ;   /* S_t */
                size_t row = ((size_t)b * L + t) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv;
                const double *dot = d_o + row * dv;
                double al = alpha[row], be = beta[row];
                /* o_t = S_t^T q_t */
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += qt[i] * dot[j];
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j) acc += St[(size_t)i * dv + j] * dot[j];
                    dq[row * dk + i] = acc;
                }
                /* a = S_{t-1}^T k_t, u, du = G^T k_t */
                for (int j = 0; j < dv; ++j) {
                    double acc = 0.0, acc2 = 0.0;
                    for (int i = 0; i < dk; ++i) {
                        acc += kt[i] * Sp[(size_t)i * dv + j];
                        acc2 += kt[i] * G[(size_t)i * dv + j];
                    }
                    a[j] = acc;
                    u[j] = be * (vt[j] - al * acc);
                    du[j] = acc2;
                }
                double db = 0.0, dal = 0.0, dua = 0.0;
                for (int j = 0; j < dv; ++j) {
                    dvv[row * dv + j] = be * du[j];
                    db += du[j] * (vt[j] - al * a[j]);
                    dua += du[j] * a[j];
                }
                for (int i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dv; ++j)
                        acc += G[(size_t)i * dv + j] * u[j] - al * be * Sp[(size_t)i * dv + j] * du[j];
                    dkk[row * dk + i] = acc;
                    for (int j = 0; j < dv; ++j) dal += G[(size_t)i * dv + j] * Sp[(size_t)i * dv + j];
                }
                dbeta[row] = db;
                dalpha[row] = dal - be * dua;
                /* G <- dL/dS_{t-1} */
                for (int i = 0; i < dk; ++i)
                    for (int j = 0; j < dv; ++j)
                        G[(size_t)i * dv + j] = al * G[(size_t)i * dv + j] - al * be * kt[i] * du[j];
            }
        }
        if (ds_init) memcpy(ds_init + (size_t)p * SZ, G, sizeof(double) * SZ);
#undef STEP
        free(ck); free(hist); free(G); free(vec);
    }
    return failed ? -1 : 0;
}
