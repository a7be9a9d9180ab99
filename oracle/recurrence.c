/*
 * fp64 token recurrence for causal decayed linear attention, in plain C.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg through oracle/crec.py; never by the product
 * path.  It shares no code with the HIP library.
 *
 * Per (batch, head) pair, with decay lam (the MiniMax-M1 fact sheet, archdb,
 * "linear / SSM layer configuration" field: fixed per-head exponential decay,
 * d x d state per head):
 *
 *     S_{-1} = S0 (or 0),   S_t = lam * S_{t-1} + k_t^T v_t,   o_t = q_t S_t
 *
 * The state is S[key][value], row-major.  Inputs are fp32 arrays (bf16 data
 * embeds exactly); every operation runs in double.  Pairs are independent and
 * are spread over OpenMP threads; nothing else is reordered.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int lcd_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * q, k, v      : [pairs][n][d] float
 * lam          : [pairs] double (the decay of each pair's head)
 * s0           : [pairs][d][d] double, or NULL for a zero initial state
 * o            : [pairs][o_to - o_from][d] double, or NULL; receives o_t for
 *                o_from <= t < o_to
 * s_final      : [pairs][d][d] double, or NULL; receives S_{n-1} (S0 if n == 0)
 * nthreads     : OpenMP threads to use (<= 0: the runtime's default)
 * Returns 0, or -1 if a scratch allocation failed.
 */
int lcd_oracle_recurrent(const float *q, const float *k, const float *v,
                         const double *lam, const double *s0,
                         double *o, int64_t o_from, int64_t o_to,
                         double *s_final,
                         int64_t pairs, int64_t n, int64_t d, int nthreads)
{
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        double *S = (double *)malloc(sizeof(double) * (size_t)(d * d));
        double *acc = (double *)malloc(sizeof(double) * (size_t)d);
        if (!S || !acc) {
            free(S);
            free(acc);
            failed = 1;
            continue;
        }
        if (s0)
            memcpy(S, s0 + p * d * d, sizeof(double) * (size_t)(d * d));
        else
            memset(S, 0, sizeof(double) * (size_t)(d * d));
        const double lm = lam[p];
        const float *qp = q + p * n * d, *kp = k + p * n * d, *vp = v + p * n * d;
        for (int64_t t = 0; t < n; ++t) {
            const float *qt = qp + t * d, *kt = kp + t * d, *vt = vp + t * d;
            for (int64_t j = 0; j < d; ++j) acc[j] = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                const double ki = (double)kt[i];
                const double qi = (double)qt[i];
                double *Si = S + i * d;
                for (int64_t j = 0; j < d; ++j) {
                    const double s = lm * Si[j] + ki * (double)vt[j];
                    Si[j] = s;
                    acc[j] += qi * s;
                }
            }
            if (o && t >= o_from && t < o_to) {
                double *ot = o + (p * (o_to - o_from) + (t - o_from)) * d;
                for (int64_t j = 0; j < d; ++j) ot[j] = acc[j];
            }
        }
        if (s_final) memcpy(s_final + p * d * d, S, sizeof(double) * (size_t)(d * d));
        free(S);
        free(acc);
    }
    return failed ? -1 : 0;
}

/*
 * Gradients of the recurrence above for a loss L whose gradient with respect
 * to the outputs is dout (dL/do_t) and with respect to the final state
 * S_{n-1} is dsn (NULL = 0), per pair:
 *
 *   forward   S_t = lam S_{t-1} + k_t^T v_t,        dq_t = dout_t S_t^T
 *   adjoint   G_t = dL/dS_t, taken from the last token back:
 *             G_{n-1} = dsn + q_{n-1}^T dout_{n-1},  G_t = lam G_{t+1} + q_t^T dout_t
 *             dk_t = v_t G_t^T,  dv_t = k_t G_t
 *   initial   ds0 = dL/dS_{-1} = lam G_0   (dsn itself when n == 0)
 *
 * q, k, v, dout : [pairs][n][d] float;  lam : [pairs] double
 * s0, dsn       : [pairs][d][d] double or NULL (zero)
 * dq, dk, dv    : [pairs][n][d] double (written);  ds0 : [pairs][d][d] double or NULL
 * Returns 0, or -1 if a scratch allocation failed.
 */
int lcd_oracle_backward(const float *q, const float *k, const float *v, const double *lam,
                        const double *s0, const float *dout, const double *dsn,
                        double *dq, double *dk, double *dv, double *ds0,
                        int64_t pairs, int64_t n, int64_t d, int nthreads)
{
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t p = 0; p < pairs; ++p) {
        double *S = (double *)malloc(sizeof(double) * (size_t)(d * d));
        if (!S) {
            failed = 1;
            continue;
        }
        const double lm = lam[p];
        const float *qp = q + p * n * d, *kp = k + p * n * d, *vp = v + p * n * d, *gp = dout + p * n * d;
        /* forward: the states S_t, and dq_t = dout_t S_t^T */
        if (s0)
            memcpy(S, s0 + p * d * d, sizeof(double) * (size_t)(d * d));
        else
            memset(S, 0, sizeof(double) * (size_t)(d * d));
        for (int64_t t = 0; t < n; ++t) {
            const float *kt = kp + t * d, *vt = vp + t * d, *gt = gp + t * d;
            double *dqt = dq + (p * n + t) * d;
            for (int64_t i = 0; i < d; ++i) {
                double *Si = S + i * d;
                double acc = 0.0;
                for (int64_t j = 0; j < d; ++j) {
                    Si[j] = lm * Si[j] + (double)kt[i] * (double)vt[j];
                    acc += (double)gt[j] * Si[j];
                }
                dqt[i] = acc;
            }
        }
        /* adjoint, last token first: S now holds G */
        if (dsn)
            memcpy(S, dsn + p * d * d, sizeof(double) * (size_t)(d * d));
        else
            memset(S, 0, sizeof(double) * (size_t)(d * d));
        for (int64_t t = n - 1; t >= 0; --t) {
            const float *qt = qp + t * d, *kt = kp + t * d, *vt = vp + t * d, *gt = gp + t * d;
            const double f = (t == n - 1) ? 1.0 : lm;
            double *dkt = dk + (p * n + t) * d, *dvt = dv + (p * n + t) * d;
            for (int64_t j = 0; j < d; ++j) dvt[j] = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                double *Gi = S + i * d;
                double acc = 0.0;
                for (int64_t j = 0; j < d; ++j) {
                    Gi[j] = f * Gi[j] + (double)qt[i] * (double)gt[j];
                    acc += Gi[j] * (double)vt[j];
                    dvt[j] += (double)kt[i] * Gi[j];
                }
                dkt[i] = acc;
            }
        }
        if (ds0) {
            double *dsp = ds0 + p * d * d;
            const double f = (n > 0) ? lm : 1.0;
            for (int64_t e = 0; e < d * d; ++e) dsp[e] = f * S[e];
        }
        free(S);
    }
    return failed ? -1 : 0;
}
