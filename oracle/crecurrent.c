/*
 * Plain C float64 token recurrence for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite for full-tensor checks at
 * medium sizes and by the benchmark's CPU-baseline leg.  Shares no code with the
 * HIP path.
 *
 * Follows "Linear Attention Sequence Parallelism" (arXiv 2404.02882), Sec. 3.2:
 *   forward  (Eq. 5):  kv_p = lam kv_{p-1} + k_p^T v_p  (kv_{-1} = M_in),  o_p = q_p kv_p
 *   backward (Eq. 12): dq_p = do_p kv_p^T,  dk_p = v_p dkv_p^T,  dv_p = k_p dkv_p
 *            (Eq. 13): dkv_p = lam dkv_{p+1} + q_p^T do_p, seeded with dM_out,
 *   and dM_in = lam dkv_0 (the gradient carried to the state before token 0).
 *
 * One "unit" is one head of one sequence: rows [row_off, row_off + len) of the
 * row-major [rows, d] input arrays.  Units run in parallel (OpenMP); each unit is
 * a plain serial loop over its tokens.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static void unit_fwd(int d, int64_t L, double lam, const float *q, const float *k,
                     const float *v, const double *m_in, double *o, double *m_out,
                     double *kv)
{
    if (m_in) memcpy(kv, m_in, sizeof(double) * d * d);
    else memset(kv, 0, sizeof(double) * d * d);
    for (int64_t p = 0; p < L; ++p) {
        const float *kp = k + p * d, *vp = v + p * d, *qp = q + p * d;
        for (int i = 0; i < d; ++i) {
            double ki = kp[i];
            double *row = kv + (int64_t)i * d;
            for (int j = 0; j < d; ++j) row[j] = lam * row[j] + ki * (double)vp[j];
        }
        if (o) {
            double *op = o + p * d;
            for (int j = 0; j < d; ++j) op[j] = 0.0;
            for (int i = 0; i < d; ++i) {
                double qi = qp[i];
                const double *row = kv + (int64_t)i * d;
                for (int j = 0; j < d; ++j) op[j] += qi * row[j];
            }
        }
    }
    if (m_out) memcpy(m_out, kv, sizeof(double) * d * d);
}

static void unit_bwd(int d, int64_t L, double lam, const float *q, const float *k,
                     const float *v, const float *dO, const double *m_in,
                     const double *dm_out, double *dq, double *dk, double *dv,
                     double *dm_in, double *kv)
{
    /* forward sweep: recompute kv_p and dq_p = do_p kv_p^T */
    if (m_in) memcpy(kv, m_in, sizeof(double) * d * d);
    else memset(kv, 0, sizeof(double) * d * d);
    for (int64_t p = 0; p < L; ++p) {
        const float *kp = k + p * d, *vp = v + p * d, *dop = dO + p * d;
        double *dqp = dq + p * d;
        for (int i = 0; i < d; ++i) {
            double ki = kp[i], acc = 0.0;
            double *row = kv + (int64_t)i * d;
            for (int j = 0; j < d; ++j) {
                row[j] = lam * row[j] + ki * (double)vp[j];
                acc += (double)dop[j] * row[j];
            }
            dqp[i] = acc;                 /* (do_p kv_p^T)_i = sum_j do_pj kv_p[i][j] */
        }
    }
    /* reverse sweep: g = dkv_p */
    double *g = kv;
    if (dm_out) memcpy(g, dm_out, sizeof(double) * d * d);
    else memset(g, 0, sizeof(double) * d * d);
    for (int64_t p = L - 1; p >= 0; --p) {
        const float *qp = q + p * d, *kp = k + p * d, *vp = v + p * d, *dop = dO + p * d;
        double *dkp = dk + p * d, *dvp = dv + p * d;
        for (int j = 0; j < d; ++j) dvp[j] = 0.0;
        for (int i = 0; i < d; ++i) {
            double qi = qp[i], ki = kp[i], acc = 0.0;
            double *row = g + (int64_t)i * d;
            for (int j = 0; j < d; ++j) {
                row[j] += qi * (double)dop[j];
                acc += (double)vp[j] * row[j];     /* (v_p g^T)_i */
                dvp[j] += ki * row[j];             /* (k_p g)_j   */
            }
            dkp[i] = acc;
        }
        for (int64_t e = 0; e < (int64_t)d * d; ++e) g[e] *= lam;
    }
    if (dm_in) memcpy(dm_in, g, sizeof(double) * d * d);
}

/* Forward (and optionally backward) over n units.  Any output pointer may be
 * NULL, then it is not written.  Returns 0, or -1 if scratch allocation fails. */
int lasp_ref_run(int n, const int64_t *row_off, const int64_t *len, const double *lam,
                 int d, const float *Q, const float *K, const float *V, const float *dO,
                 const double *m_in, const double *dm_out,
                 double *O, double *m_out, double *dQ, double *dK, double *dV,
                 double *dm_in, int do_bwd)
{
    int err = 0;
    const int64_t dd = (int64_t)d * d;
#pragma omp parallel
    {
        double *kv = (double *)malloc(sizeof(double) * dd);
        if (!kv) {
#pragma omp atomic write
            err = -1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int u = 0; u < n; ++u) {
            if (!kv) continue;
            const int64_t r = row_off[u] * d;
            const double *mi = m_in ? m_in + u * dd : NULL;
            if (O || m_out)
                unit_fwd(d, len[u], lam[u], Q + r, K + r, V + r, mi,
                         O ? O + r : NULL, m_out ? m_out + u * dd : NULL, kv);
            if (do_bwd)
                unit_bwd(d, len[u], lam[u], Q + r, K + r, V + r, dO + r, mi,
                         dm_out ? dm_out + u * dd : NULL, dQ + r, dK + r, dV + r,
                         dm_in ? dm_in + u * dd : NULL, kv);
        }
        free(kv);
    }
    return err;
}

int lasp_ref_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
