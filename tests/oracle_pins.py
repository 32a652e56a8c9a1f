"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Source: "xLSTM: Extended Long Short-Term Memory" (arXiv 2405.04517).
Every pin is a function ``pin_*(orc)`` taking an ``oracle.Oracle``; it raises
AssertionError when the oracle disagrees.  None of them retypes the oracle's
stabilized recurrence: each compares it with a different formulation whose
equality the pages or plain algebra guarantee:

* the unstabilized recurrence (section 2.2: replacing f, i by the stabilized
  f', i' changes no output; section 2.3: threshold 1.0 on |n^T q|);
* the quadratic parallel form (section 2.3: without memory mixing the
  recurrence can be rewritten in parallel form), written with numpy's own
  log-sigmoid (``-logaddexp(0, -x)``) and masked matrix products;
* eq. (18) itself (no decay, unit learning rate): C_S = V^T K by library GEMM;
* causal linear attention (eq. (18) with unit gates, the fast-weight reading of
  section 2.3) by masked matrix products;
* closed forms of a single step, of the memoryless case and of one-pair
  associative retrieval (section 2.3, the bidirectional associative memory
  setting: a stored value is retrieved by a later query along its key);
* head independence (section 2.3: no memory mixing across heads).

The backward (``Oracle.bwd``, the derivative of the quadratic form written out)
is pinned against central finite differences of the *recurrent* forward -- a
different formulation -- in both regimes of the normalizer floor, and by its
linearity in the incoming gradient.
"""
from __future__ import annotations

import numpy as np

RTOL = 1e-10


def _sig(x):
    return 1.0 / (1.0 + np.exp(-x))


def _log_sig(x):
    # numpy's own stable evaluation, independent of the oracle's formula
    return -np.logaddexp(0.0, -np.asarray(x, dtype=np.float64))


def _close(a, b, rtol=RTOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: oracle produced non-finite values"
    scale = max(float(np.max(np.abs(b))), 1e-300)
    err = float(np.max(np.abs(a - b))) / scale
    assert err <= rtol, f"{what}: max abs diff / max|ref| = {err:.3e} > {rtol:.1e}"


def _inputs(rng, B, NH, S, dqk, dv, i_mu=0.0, i_sd=1.0, f_mu=1.0, f_sd=1.5):
    q = rng.standard_normal((B, NH, S, dqk))
    k = rng.standard_normal((B, NH, S, dqk)) / np.sqrt(dqk)
    v = rng.standard_normal((B, NH, S, dv))
    i = i_mu + i_sd * rng.standard_normal((B, NH, S))
    f = f_mu + f_sd * rng.standard_normal((B, NH, S))
    o = rng.standard_normal((B, NH, S, dv))
    return q, k, v, i, f, o


# --------------------------------------------------------------------------
# independent formulations
# --------------------------------------------------------------------------
def unstabilized(q, k, v, i, f, o, C0=None, n0=None):
    """Unstabilized recurrence: f = sigmoid, i = exp, threshold 1.0 on |n.q|."""
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    h = np.zeros((B, NH, S, dv))
    Cs = np.zeros((B, NH, dv, dqk))
    ns = np.zeros((B, NH, dqk))
    nqs = np.zeros((B, NH, S))
    for b in range(B):
        for hd in range(NH):
            C = np.zeros((dv, dqk)) if C0 is None else C0[b, hd].copy()
            n = np.zeros(dqk) if n0 is None else n0[b, hd].copy()
            for t in range(S):
                fg = _sig(f[b, hd, t])
                ig = np.exp(i[b, hd, t])
                C = fg * C + ig * np.outer(v[b, hd, t], k[b, hd, t])
                n = fg * n + ig * k[b, hd, t]
                nq = n @ q[b, hd, t]
                nqs[b, hd, t] = nq
                h[b, hd, t] = _sig(o[b, hd, t]) * (C @ q[b, hd, t]) / max(abs(nq), 1.0)
            Cs[b, hd], ns[b, hd] = C, n
    return h, Cs, ns, nqs


def stabilizer_closed_form(i, f, m0=None):
    """m_t = max(m_0 + F_t, max_{s<=t} (i_s + F_t - F_s)), F = cumsum(log sigmoid(f))."""
    B, NH, S = i.shape
    F = np.cumsum(_log_sig(f), axis=-1)
    m = np.empty((B, NH, S))
    base = np.zeros((B, NH)) if m0 is None else np.asarray(m0, dtype=np.float64)
    for t in range(S):
        cand = i[..., : t + 1] + F[..., t : t + 1] - F[..., : t + 1]
        m[..., t] = np.maximum(base + F[..., t], cand.max(axis=-1))
    return m


def parallel_form(q, k, v, i, f, o, C0=None, n0=None, m0=None):
    """Quadratic (attention-like) parallel form of the whole sequence, per head.

    With F_t the cumulative log forget gate and m_t the stabilizer, the decay
    matrix is D_ts = exp(i_s + F_t - F_s - m_t) for s <= t (0 above the
    diagonal) and the initial state enters with weight g_t = exp(m_0 + F_t - m_t).
    """
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    if C0 is None:
        C0 = np.zeros((B, NH, dv, dqk))
        n0 = np.zeros((B, NH, dqk))
        m0 = np.zeros((B, NH))
    m = stabilizer_closed_form(i, f, m0)
    F = np.cumsum(_log_sig(f), axis=-1)
    h = np.empty((B, NH, S, dv))
    Cf = np.empty((B, NH, dv, dqk))
    nf = np.empty((B, NH, dqk))
    for b in range(B):
        for hd in range(NH):
            Fb, ib, mb = F[b, hd], i[b, hd], m[b, hd]
            logD = ib[None, :] + Fb[:, None] - Fb[None, :] - mb[:, None]
            mask = np.tril(np.ones((S, S), dtype=bool))
            D = np.where(mask, np.exp(np.where(mask, logD, 0.0)), 0.0)
            g = np.exp(m0[b, hd] + Fb - mb)
            Q, K, V = q[b, hd], k[b, hd], v[b, hd]
            P = (Q @ K.T) * D
            num = P @ V + g[:, None] * (Q @ C0[b, hd].T)
            den = P.sum(axis=1) + g * (Q @ n0[b, hd])
            h[b, hd] = _sig(o[b, hd]) * num / np.maximum(np.abs(den), np.exp(-mb))[:, None]
            w = np.exp(ib + Fb[-1] - Fb - mb[-1])
            a = np.exp(m0[b, hd] + Fb[-1] - mb[-1])
            Cf[b, hd] = (V * w[:, None]).T @ K + a * C0[b, hd]
            nf[b, hd] = K.T @ w + a * n0[b, hd]
    return h, Cf, nf, m[..., -1].copy()


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_stabilizer_invariance(orc):
    """Stabilized outputs equal the unstabilized ones; C' e^m = C, n' e^m = n."""
    rng = np.random.default_rng(11)
    q, k, v, i, f, o = _inputs(rng, 1, 2, 12, 3, 5)
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    hu, Cu, nu, nq = unstabilized(q, k, v, i, f, o)
    # both branches of the normalizer floor must be exercised
    assert np.any(np.abs(nq) < 1.0) and np.any(np.abs(nq) > 1.0)
    _close(h, hu, what="h vs unstabilized")
    _close(C * np.exp(m)[..., None, None], Cu, what="C' e^m vs C")
    _close(n * np.exp(m)[..., None], nu, what="n' e^m vs n")


def pin_parallel_form(orc):
    """Recurrent form equals the quadratic parallel form (zero initial state)."""
    rng = np.random.default_rng(12)
    q, k, v, i, f, o = _inputs(rng, 2, 2, 40, 6, 5, i_sd=2.0, f_mu=2.0, f_sd=2.0)
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    hp, Cp, np_, mp = parallel_form(q, k, v, i, f, o)
    _close(h, hp, what="h")
    _close(C, Cp, what="C'")
    _close(n, np_, what="n'")
    _close(m, mp, what="m")


def pin_parallel_form_initial_state(orc):
    """Recurrent form from a given stabilized state equals the parallel form."""
    rng = np.random.default_rng(13)
    q, k, v, i, f, o = _inputs(rng, 1, 3, 24, 5, 4, i_sd=1.5)
    C0 = rng.standard_normal((1, 3, 4, 5)) * 0.3
    n0 = rng.standard_normal((1, 3, 5))
    m0 = rng.uniform(-2.0, 5.0, (1, 3))
    h, C, n, m = orc.fwd(q, k, v, i, f, o, C0, n0, m0)
    hp, Cp, np_, mp = parallel_form(q, k, v, i, f, o, C0, n0, m0)
    _close(h, hp, what="h")
    _close(C, Cp, what="C'")
    _close(n, np_, what="n'")
    _close(m, mp, what="m")


def pin_extreme_gates(orc):
    """Huge gate pre-activations stay finite and still match the parallel form."""
    rng = np.random.default_rng(14)
    q, k, v, i, f, o = _inputs(rng, 1, 2, 32, 4, 4, i_sd=8.0, f_mu=1.0, f_sd=2.0)
    f[0, 0, 5] = -800.0
    f[0, 1, 9] = 800.0
    f[0, 0, 20] = -60.0
    i[0, 0, 3] = 40.0
    i[0, 1, 17] = 40.0
    i[0, 1, 2] = -300.0
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    hp, Cp, np_, mp = parallel_form(q, k, v, i, f, o)
    _close(h, hp, what="h")
    _close(C, Cp, what="C'")
    _close(n, np_, what="n'")
    _close(m, mp, what="m")


def pin_deep_forget_after_spike(orc):
    """A forget pre-activation far below the fp64 range of sigmoid still decays
    a memory written with a larger input gate (log-domain gating keeps it)."""
    rng = np.random.default_rng(23)
    q, k, v, i, f, o = _inputs(rng, 1, 2, 6, 3, 4)
    i[0, 0, 0] = 800.0
    f[0, 0, 1] = -750.0      # sigmoid underflows, log sigmoid is -750 exactly
    i[0, 1, 1] = 720.0
    f[0, 1, 2] = -715.0
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    hp, Cp, np_, mp = parallel_form(q, k, v, i, f, o)
    _close(h, hp, what="h")
    _close(C, Cp, what="C'")
    _close(n, np_, what="n'")
    _close(m, mp, what="m")


def pin_stabilizer_every_step(orc):
    """The returned m after every prefix equals the unrolled closed form."""
    rng = np.random.default_rng(15)
    q, k, v, i, f, o = _inputs(rng, 1, 2, 16, 3, 3, i_sd=3.0, f_mu=0.0, f_sd=3.0)
    mc = stabilizer_closed_form(i, f)
    for t in range(1, 17):
        _, _, _, m = orc.fwd(q[:, :, :t], k[:, :, :t], v[:, :, :t], i[:, :, :t], f[:, :, :t], o[:, :, :t])
        _close(m, mc[..., t - 1], what=f"m after {t} steps")


def pin_eq18_accumulation(orc):
    """eq. (18): no decay (f~ = +inf) and i~ = 0 give C_S = V^T K, n_S = sum k, m = 0."""
    rng = np.random.default_rng(16)
    q, k, v, _, _, o = _inputs(rng, 2, 1, 9, 4, 6)
    i = np.zeros((2, 1, 9))
    f = np.full((2, 1, 9), np.inf)
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    for b in range(2):
        _close(C[b, 0], v[b, 0].T @ k[b, 0], what="C vs V^T K")
        _close(n[b, 0], k[b, 0].sum(axis=0), what="n vs sum k")
    assert np.all(m == 0.0)


def pin_causal_linear_attention(orc):
    """Unit gates reduce retrieval to causal linear attention with |.| floor 1."""
    rng = np.random.default_rng(17)
    q, k, v, _, _, o = _inputs(rng, 1, 2, 20, 5, 3)
    i = np.zeros((1, 2, 20))
    f = np.full((1, 2, 20), np.inf)
    h, _, _, _ = orc.fwd(q, k, v, i, f, o)
    for hd in range(2):
        A = np.tril(q[0, hd] @ k[0, hd].T)
        num = A @ v[0, hd]
        den = np.maximum(np.abs(A.sum(axis=1)), 1.0)
        _close(h[0, hd], _sig(o[0, hd]) * num / den[:, None], what="h vs linear attention")


def pin_single_step(orc):
    """One step from the zero state has a closed form independent of f~."""
    rng = np.random.default_rng(18)
    q, k, v, i, f, o = _inputs(rng, 1, 6, 1, 4, 3, i_sd=2.0)
    f[0, :, 0] = [-50.0, -2.0, 0.0, 1.5, 7.0, 60.0]
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    for hd in range(6):
        kq = k[0, hd, 0] @ q[0, hd, 0]
        ei = np.exp(i[0, hd, 0])
        ref = _sig(o[0, hd, 0]) * v[0, hd, 0] * kq * ei / max(ei * abs(kq), 1.0)
        _close(h[0, hd, 0], ref, what="h_1")
        m1 = max(_log_sig(f[0, hd, 0]), i[0, hd, 0])
        _close(m[0, hd], m1, what="m_1")
        _close(C[0, hd], np.exp(i[0, hd, 0] - m1) * np.outer(v[0, hd, 0], k[0, hd, 0]), what="C'_1")
        _close(n[0, hd], np.exp(i[0, hd, 0] - m1) * k[0, hd, 0], what="n'_1")


def pin_memoryless(orc):
    """A closed forget gate (f~ = -inf) forgets everything before the current token."""
    rng = np.random.default_rng(19)
    q, k, v, i, _, o = _inputs(rng, 1, 2, 10, 4, 5, i_sd=2.0)
    f = np.full((1, 2, 10), -np.inf)
    h, _, _, m = orc.fwd(q, k, v, i, f, o)
    kq = np.einsum("bhtd,bhtd->bht", k, q)
    ei = np.exp(i)
    ref = _sig(o) * v * (kq * ei / np.maximum(ei * np.abs(kq), 1.0))[..., None]
    _close(h, ref, what="memoryless h")
    _close(m, i[..., -1], what="memoryless m")


def pin_associative_retrieval(orc):
    """One stored (k, v) pair is retrieved by later queries along +-k."""
    rng = np.random.default_rng(20)
    dqk, dv, S = 4, 5, 6
    key = rng.standard_normal(dqk)
    key /= np.linalg.norm(key)
    val = rng.standard_normal(dv)
    q = np.zeros((1, 2, S, dqk))
    k = np.zeros((1, 2, S, dqk))
    v = np.zeros((1, 2, S, dv))
    k[0, :, 0] = key
    v[0, :, 0] = val
    i = np.full((1, 2, S), -np.inf)
    i[0, 0, 0] = 2.0      # e^2 |k.q| >= 1: retrieval is normalized to +-v
    i[0, 1, 0] = -3.0     # e^-3 |k.q| < 1: the floor binds, output scales with k.q
    f = np.full((1, 2, S), np.inf)
    o = rng.standard_normal((1, 2, S, dv))
    signs = np.array([1.0, -1.0, 2.0, -0.5, 1.0, 3.0])
    q[0, :, :] = signs[:, None] * key[None, :]
    h, _, _, _ = orc.fwd(q, k, v, i, f, o)
    for t in range(S):
        _close(h[0, 0, t], _sig(o[0, 0, t]) * val * np.sign(signs[t]), what=f"retrieval head0 t={t}")
        kq = signs[t]
        ref = _sig(o[0, 1, t]) * val * kq * np.exp(-3.0) / max(np.exp(-3.0) * abs(kq), 1.0)
        _close(h[0, 1, t], ref, what=f"retrieval head1 t={t}")


def pin_head_independence(orc):
    """Heads and batch entries are independent recurrences (no memory mixing)."""
    rng = np.random.default_rng(21)
    q, k, v, i, f, o = _inputs(rng, 2, 3, 7, 3, 4)
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    for b in range(2):
        for hd in range(3):
            sl = (slice(b, b + 1), slice(hd, hd + 1))
            hs, Cs, ns, ms = orc.fwd(q[sl], k[sl], v[sl], i[sl], f[sl], o[sl])
            assert np.array_equal(hs[0, 0], h[b, hd]) and np.array_equal(Cs[0, 0], C[b, hd])
            assert np.array_equal(ns[0, 0], n[b, hd]) and np.array_equal(ms[0, 0], m[b, hd])


def pin_step_continues_fwd(orc):
    """fwd over S tokens equals fwd over a prefix followed by one-token steps."""
    rng = np.random.default_rng(22)
    q, k, v, i, f, o = _inputs(rng, 1, 2, 10, 4, 3, i_sd=2.0)
    h, C, n, m = orc.fwd(q, k, v, i, f, o)
    hp, Cs, ns, ms = orc.fwd(q[:, :, :6], k[:, :, :6], v[:, :, :6], i[:, :, :6], f[:, :, :6], o[:, :, :6])
    _close(hp, h[:, :, :6], rtol=0.0, what="prefix h")
    for t in range(6, 10):
        ht, Cs, ns, ms = orc.step(q[:, :, t], k[:, :, t], v[:, :, t], i[:, :, t], f[:, :, t], o[:, :, t], Cs, ns, ms)
        _close(ht, h[:, :, t], rtol=1e-13, what=f"step h t={t}")
    _close(Cs, C, rtol=1e-13, what="C after steps")
    _close(ns, n, rtol=1e-13, what="n after steps")
    _close(ms, m, rtol=1e-13, what="m after steps")


def _fd_case(seed, i_shift, S=7, dqk=4, dv=3, B=1, NH=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, NH, S, dqk))
    k = rng.standard_normal((B, NH, S, dqk)) / 2
    v = rng.standard_normal((B, NH, S, dv))
    i = rng.standard_normal((B, NH, S)) + i_shift
    f = 2.0 * rng.standard_normal((B, NH, S)) + 1.0
    o = rng.standard_normal((B, NH, S, dv))
    dh = rng.standard_normal((B, NH, S, dv))
    return [q, k, v, i, f, o], dh


def _finite_differences(orc, args, dh, eps=1e-6):
    """Central differences of sum(dh * h) through the recurrent forward, every input element."""
    def loss(a):
        return float(np.sum(orc.fwd(*a)[0] * dh))
    grads = []
    for ai in range(len(args)):
        g = np.zeros_like(args[ai])
        for idx in np.ndindex(*args[ai].shape):
            a = [x.copy() for x in args]
            a[ai][idx] += eps
            up = loss(a)
            a[ai][idx] -= 2 * eps
            g[idx] = (up - loss(a)) / (2 * eps)
        grads.append(g)
    return grads


def _check_bwd_fd(orc, i_shift, seed):
    args, dh = _fd_case(seed, i_shift)
    got = orc.bwd(*args, dh)
    want = _finite_differences(orc, args, dh)
    for name, g, w in zip(("dq", "dk", "dv", "di", "df", "do"), got, want):
        scale = max(float(np.max(np.abs(w))), 1e-12)
        err = float(np.max(np.abs(g - w))) / scale
        assert err < 1e-5, f"{name}: backward differs from finite differences by {err:.2e}"


def pin_bwd_finite_differences_floor_inactive(orc):
    # large input gates: |n . q| far above the floor, so the normalizer's derivative is live
    _check_bwd_fd(orc, i_shift=4.0, seed=71)


def pin_bwd_finite_differences_floor_active(orc):
    # very negative input gates: the floor max(|n . q|, 1) is active everywhere
    _check_bwd_fd(orc, i_shift=-6.0, seed=72)


def pin_bwd_linear_in_dh(orc):
    args, dh = _fd_case(73, 1.0, S=9)
    rng = np.random.default_rng(74)
    dh2 = rng.standard_normal(dh.shape)
    g1, g2 = orc.bwd(*args, dh), orc.bwd(*args, dh2)
    g12 = orc.bwd(*args, 2.0 * dh - 3.0 * dh2)
    for a, b, c in zip(g1, g2, g12):
        _close(c, 2.0 * a - 3.0 * b, rtol=1e-11, what="linearity in dh")


# ---- mLSTM block epilogue (Figure 10 caption) --------------------------------
def _epi_case(seed, B=2, NH=3, S=5, dv=8):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((B, NH, S, dv)) * 2.0 + 0.5
    x = rng.standard_normal((B, NH, S, dv))
    z = rng.standard_normal((B, NH, S, dv)) * 2.0
    gw = 1.0 + 0.3 * rng.standard_normal((NH, dv))
    gb = 0.3 * rng.standard_normal((NH, dv))
    sw = 1.0 + 0.3 * rng.standard_normal((NH, dv))
    return h, x, z, gw, gb, sw


def pin_epilogue_library_group_norm(orc):
    """GroupNorm with one group per head is torch's group_norm over a token's NH*dv
    channels (head-major); the gate is torch's sigmoid / silu."""
    import torch
    h, x, z, gw, gb, sw = _epi_case(81)
    B, NH, S, dv = h.shape
    eps = 1e-3
    tok = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(0, 2, 1, 3).reshape(B * S, NH * dv)))
    gn = torch.nn.functional.group_norm(tok(h), NH, torch.from_numpy(gw.reshape(-1)),
                                        torch.from_numpy(gb.reshape(-1)), eps)
    pre = gn + torch.from_numpy(sw.reshape(-1)) * tok(x)
    for act, fn in ((0, torch.sigmoid), (1, torch.nn.functional.silu)):
        want = (pre * fn(tok(z))).numpy().reshape(B, S, NH, dv).transpose(0, 2, 1, 3)
        _close(orc.epilogue(h, x, z, gw, gb, sw, eps, act), want, rtol=1e-12, what=f"group_norm act={act}")


def pin_epilogue_constant_head(orc):
    """A head whose channels are all equal normalizes to zero: y = (gn_b + skip_w x) act(z)."""
    h, x, z, gw, gb, sw = _epi_case(82)
    h[:] = h[..., :1]
    sig = 1.0 / (1.0 + np.exp(-z))
    _close(orc.epilogue(h, x, z, gw, gb, sw, 1e-5, 0), (gb[None, :, None, :] + sw[None, :, None, :] * x) * sig,
           rtol=1e-12, what="constant head")


def pin_epilogue_shift_scale_invariance(orc):
    """Without eps the normalization forgets any positive scale and shift of a head's row."""
    h, x, z, gw, gb, sw = _epi_case(83)
    a = 3.7 * np.ones_like(h)
    a[:, 1] = 0.02
    y0 = orc.epilogue(h, x, z, gw, gb, sw, 0.0, 1)
    y1 = orc.epilogue(a * h - 11.0, x, z, gw, gb, sw, 0.0, 1)
    _close(y1, y0, rtol=1e-9, what="shift/scale invariance")


def pin_epilogue_swish_is_z_times_sigmoid(orc):
    """The swish-gated output is the sigmoid-gated one times z."""
    h, x, z, gw, gb, sw = _epi_case(84)
    _close(orc.epilogue(h, x, z, gw, gb, sw, 1e-5, 1), orc.epilogue(h, x, z, gw, gb, sw, 1e-5, 0) * z,
           rtol=1e-12, what="swish vs sigmoid")


EPI_PINS = [
    pin_epilogue_library_group_norm,
    pin_epilogue_constant_head,
    pin_epilogue_shift_scale_invariance,
    pin_epilogue_swish_is_z_times_sigmoid,
]


# ---- sLSTM recurrence (section 2.2) -------------------------------------------
def _slstm_case(seed, B=2, NH=2, S=12, dh=6, rscale=0.3):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, NH, S, 4, dh))
    x[..., 2, :] += 2.0                         # forget gates mostly open
    R = rscale * rng.standard_normal((NH, 4, dh, dh))
    return x, R


def pin_slstm_unstabilized(orc):
    """The stabilized recurrence equals the plain exponential-gated one (c = c' e^m, n = n' e^m)."""
    x, R = _slstm_case(91)
    B, NH, S, _, dh = x.shape
    for fe in (0, 1):
        h, c, n, m, hl = orc.slstm(x, R, fe)
        for b in range(B):
            for hd in range(NH):
                cc, nn, hh = np.zeros(dh), np.zeros(dh), np.zeros(dh)
                for t in range(S):
                    a = x[b, hd, t] + R[hd] @ hh
                    i_g = np.exp(a[1])
                    f_g = np.exp(a[2]) if fe else 1.0 / (1.0 + np.exp(-a[2]))
                    cc = f_g * cc + i_g * np.tanh(a[0])
                    nn = f_g * nn + i_g
                    hh = cc / nn / (1.0 + np.exp(-a[3]))
                    _close(h[b, hd, t], hh, rtol=1e-10, what=f"slstm h fe={fe}")
                _close(c[b, hd] * np.exp(m[b, hd]), cc, rtol=1e-10, what="slstm c")
                _close(n[b, hd] * np.exp(m[b, hd]), nn, rtol=1e-10, what="slstm n")
                _close(hl[b, hd], hh, rtol=1e-12, what="slstm last h")


def pin_slstm_constant_cell_input(orc):
    """With no mixing into the cell input and a constant cell input, c / n is the
    normalized average of one value: h_t = sigmoid(a_o,t) tanh(z~) whatever the gates do."""
    x, R = _slstm_case(92, S=20)
    x[..., 0, :] = x[:, :, :1, 0, :]
    R[:, 0] = 0.0
    h, *_ = orc.slstm(x, R, 0)
    hp = np.zeros(h.shape[:2] + h.shape[3:])
    for t in range(h.shape[2]):
        a_o = x[:, :, t, 3] + np.einsum("hrj,bhj->bhr", R[:, 3], hp)
        _close(h[:, :, t], np.tanh(x[:, :, t, 0]) / (1.0 + np.exp(-a_o)), rtol=1e-12, what="constant z")
        hp = h[:, :, t]


def pin_slstm_memoryless(orc):
    """An exponential forget gate at exp(-1e4) forgets everything: the cell is the RNN
    h_t = sigmoid(a_o) tanh(a_z), a = x + R h_{t-1}."""
    x, R = _slstm_case(93)
    x[..., 2, :] = -1e4
    R[:, 2] = 0.0
    h, *_ = orc.slstm(x, R, 1)
    hp = np.zeros(h.shape[:2] + h.shape[3:])
    for t in range(h.shape[2]):
        a = x[:, :, t] + np.einsum("hgrj,bhj->bhgr", R, hp)
        hp = np.tanh(a[:, :, 0]) / (1.0 + np.exp(-a[:, :, 3]))
        _close(h[:, :, t], hp, rtol=1e-12, what="memoryless")


def pin_slstm_heads_are_diagonal_blocks(orc):
    """NH heads of dh cells equal one head of NH*dh cells whose recurrent matrices are
    block diagonal with the heads' matrices as blocks."""
    x, R = _slstm_case(94, B=1, NH=3, dh=4)
    NH, dh = 3, 4
    h, c, n, m, hl = orc.slstm(x, R, 0)
    xb = x.transpose(0, 2, 3, 1, 4).reshape(1, 1, x.shape[2], 4, NH * dh)
    Rb = np.zeros((1, 4, NH * dh, NH * dh))
    for hd in range(NH):
        Rb[0, :, hd * dh:(hd + 1) * dh, hd * dh:(hd + 1) * dh] = R[hd]
    hb, cb, nb, mb, hlb = orc.slstm(xb, Rb, 0)
    _close(hb.reshape(1, x.shape[2], NH, dh).transpose(0, 2, 1, 3), h, rtol=1e-13, what="block diagonal h")
    _close(cb.reshape(1, NH, dh), c, rtol=1e-13, what="block diagonal c")


def pin_slstm_forget_sigmoid_as_exp(orc):
    """Without mixing into the forget gate, the sigmoid forget gate on a_f is the
    exponential one on log sigmoid(a_f)."""
    x, R = _slstm_case(95)
    R[:, 2] = 0.0
    x2 = x.copy()
    x2[..., 2, :] = -np.logaddexp(0.0, -x[..., 2, :])
    a = orc.slstm(x, R, 0)
    b = orc.slstm(x2, R, 1)
    for u, v in zip(a, b):
        _close(u, v, rtol=1e-12, what="forget sigmoid vs exp")


def pin_slstm_continuation(orc):
    """Running S1 tokens, then S2 from the returned state, equals one run of S1 + S2."""
    x, R = _slstm_case(96, S=15)
    full = orc.slstm(x, R, 0)
    first = orc.slstm(x[:, :, :6], R, 0)
    second = orc.slstm(x[:, :, 6:], R, 0, *first[1:])
    _close(np.concatenate([first[0], second[0]], axis=2), full[0], rtol=1e-12, what="continued h")
    for u, v in zip(second[1:], full[1:]):
        _close(u, v, rtol=1e-12, what="continued state")


SLSTM_PINS = [
    pin_slstm_unstabilized,
    pin_slstm_constant_cell_input,
    pin_slstm_memoryless,
    pin_slstm_heads_are_diagonal_blocks,
    pin_slstm_forget_sigmoid_as_exp,
    pin_slstm_continuation,
]


BWD_PINS = [
    pin_bwd_finite_differences_floor_inactive,
    pin_bwd_finite_differences_floor_active,
    pin_bwd_linear_in_dh,
]

ALL_PINS = [
    pin_stabilizer_invariance,
    pin_parallel_form,
    pin_parallel_form_initial_state,
    pin_extreme_gates,
    pin_deep_forget_after_spike,
    pin_stabilizer_every_step,
    pin_eq18_accumulation,
    pin_causal_linear_attention,
    pin_single_step,
    pin_memoryless,
    pin_associative_retrieval,
    pin_head_independence,
    pin_step_continues_fwd,
]
