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

/*
 * Gradients of the forward from the zero state with respect to every input,
 * given the gradient dh of a loss that depends on h only (the final state is
 * not differentiated).
 *
 * Derivative of the quadratic parallel form of the recurrence (section 2.3:
 * the recurrence and its parallel form; section 2.2: the stabilizer leaves h
 * unchanged, so no gradient flows through it).  Per head, with
 *   F_t    = sum_{j<=t} log sigmoid(f~_j)
 *   D_ts   = exp(F_t - F_s + i~_s)          (s <= t; 0 otherwise)
 *   S_ts   = q_t . k_s
 *   num_t  = sum_s D_ts S_ts v_s,   den_t = sum_s D_ts S_ts
 *   N_t    = max(|den_t|, 1),       g_t = sigmoid(o~_t),   u_t = num_t / N_t
 *   h_t    = g_t (.) u_t
 * the chain rule gives
 *   do~_t  = dh_t (.) u_t (.) g_t (.) (1 - g_t)
 *   dnum_t = dh_t (.) g_t / N_t
 *   dden_t = -sign(den_t) (dh_t (.) g_t) . num_t / N_t^2   if |den_t| > 1, else 0
 *   dA_ts  = dnum_t . v_s + dden_t                  (A_ts = D_ts S_ts)
 *   dv_s   = sum_{t>=s} D_ts S_ts dnum_t
 *   dq_t   = sum_{s<=t} dA_ts D_ts k_s,   dk_s = sum_{t>=s} dA_ts D_ts q_t
 *   dlogD_ts = dA_ts D_ts S_ts:  di~_s = sum_t dlogD_ts,  dF_t += sum_s dlogD_ts,
 *                                dF_s -= sum_t dlogD_ts
 *   dlf_j  = sum_{t>=j} dF_t,    df~_j = dlf_j sigmoid(-f~_j)
 * in fp64, unstabilized (the test inputs keep every exponent far from overflow).
 * Layouts as oracle_fwd_f64; dh like h; outputs like their inputs.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_bwd_f64(const double *q, const double *k, const double *v,
                   const double *i_pre, const double *f_pre, const double *o_pre, const double *dh,
                   int B, int NH, int S, int dqk, int dv,
                   double *dq, double *dk, double *dvv, double *di, double *df, double *dout)
{
    if (B < 0 || NH < 0 || S < 0 || dqk <= 0 || dv <= 0)
        return -1;
    if (!q || !k || !v || !i_pre || !f_pre || !o_pre || !dh || !dq || !dk || !dvv || !di || !df || !dout)
        return -1;
    const int heads = B * NH;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < heads; ++bh) {
        const size_t t0 = (size_t)bh * S;
        const double *qh = q + t0 * dqk, *kh = k + t0 * dqk, *vh = v + t0 * dv;
        const double *ih = i_pre + t0, *fh = f_pre + t0, *oh = o_pre + t0 * dv, *dhh = dh + t0 * dv;
        double *dqh = dq + t0 * dqk, *dkh = dk + t0 * dqk, *dvh = dvv + t0 * dv;
        double *dih = di + t0, *dfh = df + t0, *doh = dout + t0 * dv;
        double *F = malloc(sizeof(double) * S), *dF = calloc(S, sizeof(double));
        double *Smat = malloc(sizeof(double) * (size_t)S * S), *Dmat = malloc(sizeof(double) * (size_t)S * S);
        double *num = calloc((size_t)S * dv, sizeof(double)), *den = calloc(S, sizeof(double));
        double *dnum = malloc(sizeof(double) * (size_t)S * dv), *dden = malloc(sizeof(double) * S);
        double acc = 0.0;
        for (int t = 0; t < S; ++t) {
            acc += log_sigmoid(fh[t]);
            F[t] = acc;
        }
        /* forward: scores, decay, numerator and denominator */
        for (int t = 0; t < S; ++t)
            for (int s = 0; s <= t; ++s) {
                double dot = 0.0;
                for (int j = 0; j < dqk; ++j) dot += qh[(size_t)t * dqk + j] * kh[(size_t)s * dqk + j];
                const double d = exp(F[t] - F[s] + ih[s]);
                Smat[(size_t)t * S + s] = dot;
                Dmat[(size_t)t * S + s] = d;
                for (int r = 0; r < dv; ++r) num[(size_t)t * dv + r] += d * dot * vh[(size_t)s * dv + r];
                den[t] += d * dot;
            }
        /* output gate and normalizer */
        for (int t = 0; t < S; ++t) {
            const double N = fmax(fabs(den[t]), 1.0);
            double dun = 0.0;
            for (int r = 0; r < dv; ++r) {
                const size_t e = (size_t)t * dv + r;
                const double g = sigmoid(oh[e]);
                const double u = num[e] / N;
                doh[e] = dhh[e] * u * g * (1.0 - g);
                dnum[e] = dhh[e] * g / N;
                dun += dhh[e] * g * num[e];
            }
            dden[t] = fabs(den[t]) > 1.0 ? -(den[t] > 0 ? 1.0 : -1.0) * dun / (N * N) : 0.0;
        }
        /* scores, keys, values and the log-decay */
        memset(dqh, 0, sizeof(double) * (size_t)S * dqk);
        memset(dkh, 0, sizeof(double) * (size_t)S * dqk);
        memset(dvh, 0, sizeof(double) * (size_t)S * dv);
        memset(dih, 0, sizeof(double) * S);
        for (int t = 0; t < S; ++t)
            for (int s = 0; s <= t; ++s) {
                const double d = Dmat[(size_t)t * S + s], sc = Smat[(size_t)t * S + s];
                double dA = dden[t];
                for (int r = 0; r < dv; ++r) {
                    dA += dnum[(size_t)t * dv + r] * vh[(size_t)s * dv + r];
                    dvh[(size_t)s * dv + r] += d * sc * dnum[(size_t)t * dv + r];
                }
                for (int j = 0; j < dqk; ++j) {
                    dqh[(size_t)t * dqk + j] += dA * d * kh[(size_t)s * dqk + j];
                    dkh[(size_t)s * dqk + j] += dA * d * qh[(size_t)t * dqk + j];
                }
                const double dl = dA * d * sc;
                dih[s] += dl;
                dF[t] += dl;
                dF[s] -= dl;
            }
        /* forget gate: reverse cumulative sum, then through log sigmoid */
        double rev = 0.0;
        for (int j = S - 1; j >= 0; --j) {
            rev += dF[j];
            dfh[j] = rev * sigmoid(-fh[j]);
        }
        free(F); free(dF); free(Smat); free(Dmat); free(num); free(den); free(dnum); free(dden);
    }
    return 0;
}

/* Number of OpenMP threads a parallel region of the oracle would use. */
/*
 * mLSTM block epilogue (xLSTM paper, Figure 10 caption, the mLSTM block): the
 * cell output h of each head is normalized by a GroupNorm with one group per
 * head (a LayerNorm over that head's d_v channels, with a per-channel scale and
 * shift), the learnable skip input is added, and the sum is gated component-wise
 * by the external output gate:
 *   mu = mean_r h_r,  var = mean_r (h_r - mu)^2            (over the head's d_v)
 *   y_r = (gn_w_r (h_r - mu) / sqrt(var + eps) + gn_b_r + skip_w_r x_r) * act(z_r)
 * The caption does not name the gate's activation: act = sigmoid (act = 0) or
 * swish z sigmoid(z) (act = 1).  Per-channel parameters are [NH][dv]; h, x, z and
 * y are [B][NH][S][dv].
 */
int oracle_epilogue_f64(const double *h, const double *x, const double *z,
                        const double *gn_w, const double *gn_b, const double *skip_w,
                        int B, int NH, int S, int dv, double eps, int act, double *y)
{
    if (B < 0 || NH < 0 || S < 0 || dv <= 0 || !(eps >= 0.0) || (act != 0 && act != 1))
        return -1;
    if (!h || !x || !z || !gn_w || !gn_b || !skip_w || !y)
        return -1;
    for (int b = 0; b < B; ++b)
        for (int hd = 0; hd < NH; ++hd)
            for (int t = 0; t < S; ++t) {
                const size_t row = (((size_t)b * NH + hd) * S + t) * dv;
                const double *hr = h + row;
                double mu = 0.0;
                for (int r = 0; r < dv; ++r) mu += hr[r];
                mu /= dv;
                double var = 0.0;
                for (int r = 0; r < dv; ++r) var += (hr[r] - mu) * (hr[r] - mu);
                var /= dv;
                const double inv = 1.0 / sqrt(var + eps);
                for (int r = 0; r < dv; ++r) {
                    const size_t c = (size_t)hd * dv + r;
                    const double g = act == 0 ? sigmoid(z[row + r]) : z[row + r] * sigmoid(z[row + r]);
                    y[row + r] = (gn_w[c] * (hr[r] - mu) * inv + gn_b[c] + skip_w[c] * x[row + r]) * g;
                }
            }
    return 0;
}

/*
 * sLSTM recurrence with block-diagonal memory mixing (xLSTM paper, section 2.2:
 * exponential gating with normalizer and stabilizer states, memory mixing through
 * recurrent connections from the hidden state to the cell input and the gates,
 * mixing within a head but not across heads; section 2.1 for the LSTM cell it
 * extends).  The equations are not legible on the pages; this is the plainest
 * reading of their description.  Per (b, head), cells r = 0..dh-1:
 *   a_g = x_pre[t][g] + R_g h_{t-1}        g = z, i, f, o (R_g [dh][dh], row = output cell)
 *   log i = a_i;  log f = log sigmoid(a_f)  (forget_exp = 0)  or  a_f  (forget_exp = 1)
 *   m_t = max(log f + m_{t-1}, log i)
 *   c_t = exp(log f + m_{t-1} - m_t) c_{t-1} + exp(log i - m_t) tanh(a_z)
 *   n_t = exp(log f + m_{t-1} - m_t) n_{t-1} + exp(log i - m_t)
 *   h_t = sigmoid(a_o) c_t / n_t
 * (c, n are the stabilized states: the unstabilized ones times exp(-m_t), a factor
 * that cancels in h.)  Layouts: x_pre [B][NH][S][4][dh] (gate order z, i, f, o),
 * R [NH][4][dh][dh], states [B][NH][dh], h [B][NH][S][dh].  All of c0, n0, m0, h0
 * NULL = the zero state (c = n = m = h = 0).
 */
int oracle_slstm_f64(const double *x_pre, const double *R, int B, int NH, int S, int dh, int forget_exp,
                     const double *c0, const double *n0, const double *m0, const double *h0,
                     double *h, double *c_out, double *n_out, double *m_out, double *h_out)
{
    if (B < 0 || NH < 0 || S < 0 || dh <= 0 || (forget_exp != 0 && forget_exp != 1))
        return -1;
    if (!x_pre || !R || !h || !c_out || !n_out || !m_out || !h_out)
        return -1;
    const int given = (c0 != NULL) + (n0 != NULL) + (m0 != NULL) + (h0 != NULL);
    if (given != 0 && given != 4)
        return -1;
    const int heads = B * NH;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < heads; ++bh) {
        const int hd = bh % NH;
        const double *Rh = R + (size_t)hd * 4 * dh * dh;
        double *c = c_out + (size_t)bh * dh, *n = n_out + (size_t)bh * dh;
        double *m = m_out + (size_t)bh * dh, *hp = h_out + (size_t)bh * dh;
        for (int r = 0; r < dh; ++r) {
            c[r] = given ? c0[(size_t)bh * dh + r] : 0.0;
            n[r] = given ? n0[(size_t)bh * dh + r] : 0.0;
            m[r] = given ? m0[(size_t)bh * dh + r] : 0.0;
            hp[r] = given ? h0[(size_t)bh * dh + r] : 0.0;
        }
        double *a = malloc(sizeof(double) * 4 * dh);
        for (int t = 0; t < S; ++t) {
            const double *xt = x_pre + ((size_t)bh * S + t) * 4 * dh;
            for (int g = 0; g < 4; ++g)
                for (int r = 0; r < dh; ++r) {
                    double acc = xt[g * dh + r];
                    const double *row = Rh + ((size_t)g * dh + r) * dh;
                    for (int j = 0; j < dh; ++j) acc += row[j] * hp[j];
                    a[g * dh + r] = acc;
                }
            double *ht = h + ((size_t)bh * S + t) * dh;
            for (int r = 0; r < dh; ++r) {
                const double az = a[r], ai = a[dh + r], af = a[2 * dh + r], ao = a[3 * dh + r];
                const double log_f = forget_exp ? af : log_sigmoid(af);
                const double m_t = fmax(log_f + m[r], ai);
                const double fs = exp(log_f + m[r] - m_t), is = exp(ai - m_t);
                c[r] = fs * c[r] + is * tanh(az);
                n[r] = fs * n[r] + is;
                m[r] = m_t;
                ht[r] = sigmoid(ao) * c[r] / n[r];
            }
            for (int r = 0; r < dh; ++r) hp[r] = ht[r];
        }
        free(a);
    }
    return 0;
}

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
