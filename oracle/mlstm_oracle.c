/*
 * mlstm_oracle.c -- plain fp64 CPU oracle of the mLSTM matrix-memory cell.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file; only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg do.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it computes (xLSTM: Extended Long Short-Term Memory, arXiv 2405.04517):
 *   - section 2.3 "mLSTM", eq. (18): the covariance update C_t = C_{t-1} + v_t k_t^T,
 *     with the forget gate acting as the decay rate on C_{t-1} and the input gate
 *     as the learning rate on v_t k_t^T, while the output gate scales the
 *     retrieved vector;
 *   - section 2.3 (normalizer paragraph): the normalizer is the key vectors
 *     weighted by the input gate and all later forget gates; retrieval divides by
 *     the absolute value of n_t^T q_t, floored at a threshold of 1.0;
 *   - section 2.2 (stabilizer paragraph, eq. (17) and the sentence after it): an
 *     extra state m_t keeps the exponential gates from overflowing; replacing f_t
 *     by f'_t and i_t by i'_t leaves the outputs unchanged;
 *   - section 2.3 (multi-head paragraph): heads have no memory mixing, so each
 *     (batch, head) pair is an independent recurrence.
 * The exact stabilized recurrence (input gate exp, forget gate sigmoid):
 *   m_t  = max(log f_t + m_{t-1}, log i_t)
 *   f'_t = exp(log f_t + m_{t-1} - m_t),   i'_t = exp(log i_t - m_t)
 *   C'_t = f'_t C'_{t-1} + i'_t v_t k_t^T   (C' = C e^{-m})
 *   n'_t = f'_t n'_{t-1} + i'_t k_t         (n' = n e^{-m})
 *   h_t  = sigmoid(o~_t) (.) (C'_t q_t) / max(|n'_t . q_t|, exp(-m_t))
 * The floor exp(-m_t) on the stabilized normalizer is the threshold 1.0 on the
 * unstabilized one, since n_t = n'_t e^{m_t}.
 *
 * Readings where the pages are silent: the output gate pre-activation o~ is a
 * vector over the value dimension (the block figure applies the output gate
 * component-wise); the initial state is C'=0, n'=0, m=0 unless one is passed;
 * log sigmoid(x) is evaluated as min(x,0) - log1p(exp(-|x|)) so that it stays
 * finite for large |x|.
 *
 * Layout (row-major, contiguous): q,k [B,NH,S,dqk]; v [B,NH,S,dv];
 * i_pre,f_pre [B,NH,S]; o_pre [B,NH,S,dv]; h [B,NH,S,dv]; C [B,NH,dv,dqk]
 * (rows index value dimensions, because C accumulates v k^T); n [B,NH,dqk];
 * m [B,NH].  All fp64.  Parity of every function here is pinned by the
 * oracle tests (stabilizer invariance, eq. (18) special case, closed-form
 * single step, associative-memory retrieval, quadratic parallel form,
 * causal linear attention and memoryless special cases).
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

static double log_sigmoid(double x)
{
    return fmin(x, 0.0) - log1p(exp(-fabs(x)));
}

static double sigmoid(double x)
{
    return 1.0 / (1.0 + exp(-x));
}

/*
 * One step of the stabilized recurrence for a single head.  C is dv x dqk,
 * n is dqk, *m the stabilizer; all are updated in place.  h receives dv values.
 */
static void mlstm_cell_step(int dqk, int dv,
                            const double *q, const double *k, const double *v,
                            double i_pre, double f_pre, const double *o_pre,
                            double *C, double *n, double *m, double *h)
{
    const double log_f = log_sigmoid(f_pre);  /* forget gate: sigmoid          */
    const double log_i = i_pre;               /* input gate: exp, so log i = i~ */
    const double m_prev = *m;
    const double m_t = fmax(log_f + m_prev, log_i);
    const double f_s = exp(log_f + m_prev - m_t);   /* f'_t */
    const double i_s = exp(log_i - m_t);            /* i'_t */

    /* covariance update of the matrix memory: C' <- f' C' + i' v k^T */
    for (int r = 0; r < dv; ++r) {
        double *row = C + (size_t)r * dqk;
        for (int j = 0; j < dqk; ++j)
            row[j] = f_s * row[j] + i_s * v[r] * k[j];
    }
    /* normalizer: n' <- f' n' + i' k */
    for (int j = 0; j < dqk; ++j)
        n[j] = f_s * n[j] + i_s * k[j];

    /* retrieval with the normalizer floor */
    double nq = 0.0;
    for (int j = 0; j < dqk; ++j)
        nq += n[j] * q[j];
    const double denom = fmax(fabs(nq), exp(-m_t));
    for (int r = 0; r < dv; ++r) {
        const double *row = C + (size_t)r * dqk;
        double cq = 0.0;
        for (int j = 0; j < dqk; ++j)
            cq += row[j] * q[j];
        h[r] = sigmoid(o_pre[r]) * cq / denom;
    }
    *m = m_t;
}

/*
 * Full-sequence forward of every (batch, head), token by token.
 * C0/n0/m0 give the initial stabilized state; pass NULL for all three to start
 * from C'=0, n'=0, m=0.  Outputs h, C, n, m must not alias the inputs.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fwd_f64(const double *q, const double *k, const double *v,
                   const double *i_pre, const double *f_pre, const double *o_pre,
                   int B, int NH, int S, int dqk, int dv,
                   const double *C0, const double *n0, const double *m0,
                   double *h, double *C, double *n, double *m)
{
    if (B < 0 || NH < 0 || S < 0 || dqk <= 0 || dv <= 0)
        return -1;
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !h || !C || !n || !m)
        return -1;
    const int heads = B * NH;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < heads; ++bh) {
        double *Cb = C + (size_t)bh * dv * dqk;
        double *nb = n + (size_t)bh * dqk;
        double *mb = m + bh;
        if (C0) memcpy(Cb, C0 + (size_t)bh * dv * dqk, sizeof(double) * (size_t)dv * dqk);
        else    memset(Cb, 0, sizeof(double) * (size_t)dv * dqk);
        if (n0) memcpy(nb, n0 + (size_t)bh * dqk, sizeof(double) * (size_t)dqk);
        else    memset(nb, 0, sizeof(double) * (size_t)dqk);
        *mb = m0 ? m0[bh] : 0.0;
        for (int t = 0; t < S; ++t) {
            const size_t tok = (size_t)bh * S + t;
            mlstm_cell_step(dqk, dv,
                            q + tok * dqk, k + tok * dqk, v + tok * dv,
                            i_pre[tok], f_pre[tok], o_pre + tok * dv,
                            Cb, nb, mb, h + tok * dv);
        }
    }
    return 0;
}

/*
 * One recurrent decode step for every (batch, head): the recurrence applied once
 * to the stabilized state (C, n, m), which is updated in place.
 * q,k [B,NH,dqk]; v [B,NH,dv]; i_pre,f_pre [B,NH]; o_pre [B,NH,dv]; h [B,NH,dv].
 */
int oracle_step_f64(const double *q, const double *k, const double *v,
                    const double *i_pre, const double *f_pre, const double *o_pre,
                    int B, int NH, int dqk, int dv,
                    double *C, double *n, double *m, double *h)
{
    if (B < 0 || NH < 0 || dqk <= 0 || dv <= 0)
        return -1;
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !h || !C || !n || !m)
        return -1;
    const int heads = B * NH;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < heads; ++bh) {
        mlstm_cell_step(dqk, dv,
                        q + (size_t)bh * dqk, k + (size_t)bh * dqk, v + (size_t)bh * dv,
                        i_pre[bh], f_pre[bh], o_pre + (size_t)bh * dv,
                        C + (size_t)bh * dv * dqk, n + (size_t)bh * dqk, m + bh,
                        h + (size_t)bh * dv);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle would use. */
int oracle_num_threads(void)
{
    int nt = 1;
    #pragma omp parallel
    {
        #pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            nt = omp_get_num_threads();
#endif
        }
    }
    return nt;
}
