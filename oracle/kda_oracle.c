/*
 * fp64 CPU oracle for the Kimi Delta Attention (KDA) forward recurrence.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * What it computes is the plain definition, one token at a time, in fp64
 * (page "Yanjiu KimiK3, wo faxian damoxing zhengzai xuehui guanli ziji de
 * jisuan", http://www.pwwt.cn/news/3763336/):
 *
 *   - the state S_t is a d_k x d_v matrix mapping key space to value space
 *     (section 2.1, state definition);
 *   - KDA update (section 4, KDA update equation):
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
 *     evaluated here in its error form (section 3): first decay every key
 *     channel, S' = Diag(alpha_t) S_{t-1}; then predict v_hat = S'^T k_t;
 *     then write the error, S_t = S' + beta_t k_t (v_t - v_hat)^T.  Expanding
 *     the error form gives exactly the projection form above;
 *   - readout after the update, o_t = S_t^T q_t (section 2.1, read equation).
 *
 * With flag KDA_ORACLE_NO_CORRECTION the prediction is dropped (v_hat = 0),
 * which turns the write into S_t = Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T;
 * with alpha = 1 and beta = 1 that is the plain linear-memory write of
 * section 2.1.  It exists so tests can pin the oracle against closed forms.
 *
 * Layouts (row-major, contiguous, fp64):
 *   q, k, alpha : [B, T, H, dk]     v, o : [B, T, H, dv]     beta : [B, T, H]
 *   S0, ST      : [B, H, dk, dv]
 * S0 == NULL means a zero initial state; o == NULL or ST == NULL skip that
 * output.  ST may alias S0.  (b, h) chains are independent and run in
 * parallel with OpenMP (nthreads <= 0 keeps the OpenMP default).
 * Returns 0, or -1 on a bad argument, or -2 when memory runs out.
 */
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KDA_ORACLE_NO_CORRECTION 1

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *alpha, const double *beta, const double *S0,
                   double *o, double *ST, long B, long T, long H, long dk,
                   long dv, int flags, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk < 1 || dv < 1) return -1;
    if (T > 0 && (!q || !k || !v || !alpha || !beta)) return -1;
    const long chains = B * H;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *vhat = (double *)malloc(sizeof(double) * (size_t)dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !vhat || !e) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long c = 0; c < chains; ++c) {
                const long b = c / H, h = c % H;
                if (S0)
                    memcpy(S, S0 + c * dk * dv, sizeof(double) * (size_t)(dk * dv));
                else
                    memset(S, 0, sizeof(double) * (size_t)(dk * dv));

                for (long t = 0; t < T; ++t) {
                    const long tok = (b * T + t) * H + h; /* (b, t, h) */
                    const double *qt = q + tok * dk;
                    const double *kt = k + tok * dk;
                    const double *at = alpha + tok * dk;
                    const double *vt = v + tok * dv;
                    const double bt = beta[tok];

                    /* S' = Diag(alpha_t) S, and v_hat = S'^T k_t. */
                    for (long j = 0; j < dv; ++j) vhat[j] = 0.0;
                    for (long i = 0; i < dk; ++i) {
                        double *row = S + i * dv;
                        const double a = at[i], ki = kt[i];
                        for (long j = 0; j < dv; ++j) {
                            row[j] *= a;
                            vhat[j] += row[j] * ki;
                        }
                    }
                    /* error e = v_t - v_hat (or v_t alone without correction) */
                    for (long j = 0; j < dv; ++j)
                        e[j] = (flags & KDA_ORACLE_NO_CORRECTION) ? vt[j] : vt[j] - vhat[j];

                    /* S = S' + beta_t k_t e^T, then o_t = S^T q_t */
                    double *ot = o ? o + tok * dv : NULL;
                    if (ot)
                        for (long j = 0; j < dv; ++j) ot[j] = 0.0;
                    for (long i = 0; i < dk; ++i) {
                        double *row = S + i * dv;
                        const double w = bt * kt[i], qi = qt[i];
                        for (long j = 0; j < dv; ++j) {
                            row[j] += w * e[j];
                            if (ot) ot[j] += row[j] * qi;
                        }
                    }
                }
                if (ST)
                    memcpy(ST + c * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
            }
        }
        free(S);
        free(vhat);
        free(e);
    }
    return failed ? -2 : 0;
}

/* Number of threads an OpenMP parallel region would use (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
