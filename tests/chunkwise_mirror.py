"""fp64 numpy model of the chunkwise decomposition the bf16 MFMA forward uses.

Test-side aid only: it is not the oracle (the oracle is the token-by-token
recurrence in ``oracle/``) and the HIP path does not use it.  It lets the
algebra of the kernel's two passes be checked on the CPU against the oracle:

Pass 1, per (head, chunk), independent of every other chunk:
    b_tau       = in-chunk cumulative sum of log sigmoid(f~)
    m_loc_tau   = b_tau + max_{s<=tau} (i~_s - b_s)        (chunk-local row max)
    P_loc       = (Q K^T) (.) exp(b_tau - b_s + i~_s - m_loc_tau),  s <= tau
    den_loc_tau = rowsum(P_loc)
Pass 2, per head, sequential over chunks with the carried (C', n', m_p):
    m_tau   = max(b_tau + m_p, m_loc_tau)       (the recurrent stabilizer)
    a_tau   = exp(b_tau + m_p - m_tau),   r_tau = exp(m_loc_tau - m_tau)
    num     = r (.) (P_loc V) + a (.) (Q C'^T),  den = r (.) den_loc + a (.) (Q n')
    h       = sigmoid(o~) (.) num / max(|den|, exp(-m_tau))
    w_s     = r_L exp(b_L - b_s + i~_s - m_loc_L),   alpha = exp(b_L + m_p - m_L)
    C' <- alpha C' + (w (.) V)^T K ... stored as C'[value, key]; n' <- alpha n' + K^T w
"""
from __future__ import annotations

import numpy as np


def _log_sig(x):
    return -np.logaddexp(0.0, -x)


def pass1(q, k, i, f):
    """q,k [S,dqk]; i,f [S] for one chunk -> (b, m_loc, P_loc, den_loc)."""
    b = np.cumsum(_log_sig(f))
    m_loc = b + np.maximum.accumulate(i - b)
    L = len(b)
    logD = b[:, None] - b[None, :] + i[None, :] - m_loc[:, None]
    mask = np.tril(np.ones((L, L), dtype=bool))
    D = np.where(mask, np.exp(np.where(mask, logD, -np.inf)), 0.0)
    P = (q @ k.T) * D
    return b, m_loc, P, P.sum(axis=1)


def chunkwise_forward(q, k, v, i, f, o, chunk, C0=None, n0=None, m0=None):
    """One head: q,k [S,dqk], v,o [S,dv], i,f [S] -> h [S,dv], C' [dv,dqk], n' [dqk], m."""
    S, dqk = q.shape
    dv = v.shape[1]
    C = np.zeros((dv, dqk)) if C0 is None else C0.copy()
    n = np.zeros(dqk) if n0 is None else n0.copy()
    m_p = 0.0 if m0 is None else float(m0)
    h = np.empty((S, dv))
    for t0 in range(0, S, chunk):
        sl = slice(t0, min(S, t0 + chunk))
        Q, K, V, I, F, O = q[sl], k[sl], v[sl], i[sl], f[sl], o[sl]
        b, m_loc, P, den_loc = pass1(Q, K, I, F)
        m_t = np.maximum(b + m_p, m_loc)
        a = np.exp(b + m_p - m_t)
        r = np.exp(m_loc - m_t)
        num = r[:, None] * (P @ V) + a[:, None] * (Q @ C.T)
        den = r * den_loc + a * (Q @ n)
        h[sl] = (1.0 / (1.0 + np.exp(-O))) * num / np.maximum(np.abs(den), np.exp(-m_t))[:, None]
        w_loc = np.exp(b[-1] - b + I - m_loc[-1])
        w = r[-1] * w_loc
        alpha = np.exp(b[-1] + m_p - m_t[-1])
        C = alpha * C + (V * w[:, None]).T @ K
        n = alpha * n + K.T @ w
        m_p = m_t[-1]
    return h, C, n, m_p
