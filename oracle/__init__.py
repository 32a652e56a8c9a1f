"""fp64 CPU oracle of the mLSTM matrix-memory cell -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (``mlstm_matrix_memory_amd``)
never imports, links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``mlstm_oracle.c`` (plain C, fp64, OpenMP over the
independent heads): the stabilized mLSTM recurrence of "xLSTM: Extended Long
Short-Term Memory", section 2.3 (eq. (18), the normalizer paragraph and the
multi-head paragraph) with the stabilizer of section 2.2 (eq. (17)), the
derivative of its parallel form, the mLSTM block's epilogue (Figure 10), and
the sLSTM recurrence with block-diagonal memory mixing (section 2.2).  This module
only compiles it with gcc and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "mlstm_oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE semantics, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", output + ".tmp", source, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


def _bind(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_fwd_f64.restype = ctypes.c_int
    lib.oracle_fwd_f64.argtypes = [dp] * 6 + [ctypes.c_int] * 5 + [dp] * 3 + [dp] * 4
    lib.oracle_step_f64.restype = ctypes.c_int
    lib.oracle_step_f64.argtypes = [dp] * 6 + [ctypes.c_int] * 4 + [dp] * 4
    lib.oracle_bwd_f64.restype = ctypes.c_int
    lib.oracle_bwd_f64.argtypes = [dp] * 7 + [ctypes.c_int] * 5 + [dp] * 6
    lib.oracle_epilogue_f64.restype = ctypes.c_int
    lib.oracle_epilogue_f64.argtypes = [dp] * 6 + [ctypes.c_int] * 4 + [ctypes.c_double, ctypes.c_int, dp]
    lib.oracle_slstm_f64.restype = ctypes.c_int
    lib.oracle_slstm_f64.argtypes = [dp, dp] + [ctypes.c_int] * 5 + [dp] * 4 + [dp] * 5
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
            build()
        _lib = _bind(ctypes.CDLL(LIBRARY))
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """Thin numpy front end over one loaded oracle library."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else load()

    def fwd(self, q, k, v, i_pre, f_pre, o_pre, C0=None, n0=None, m0=None):
        """Recurrent forward.  q,k [B,NH,S,dqk], v,o_pre [B,NH,S,dv], i_pre,f_pre [B,NH,S].

        Returns (h [B,NH,S,dv], C [B,NH,dv,dqk], n [B,NH,dqk], m [B,NH]) in fp64, the
        state in stabilized form (C' = C e^{-m}, n' = n e^{-m}).
        """
        q, k, v, i_pre, f_pre, o_pre = map(_f64, (q, k, v, i_pre, f_pre, o_pre))
        B, NH, S, dqk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, NH, S, dv)
        assert i_pre.shape == (B, NH, S) and f_pre.shape == (B, NH, S)
        assert o_pre.shape == (B, NH, S, dv)
        have_state = C0 is not None
        if have_state:
            C0, n0, m0 = _f64(C0), _f64(n0), _f64(m0)
            assert C0.shape == (B, NH, dv, dqk) and n0.shape == (B, NH, dqk) and m0.shape == (B, NH)
        h = np.empty((B, NH, S, dv))
        C = np.empty((B, NH, dv, dqk))
        n = np.empty((B, NH, dqk))
        m = np.empty((B, NH))
        rc = self.lib.oracle_fwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
                                     B, NH, S, dqk, dv,
                                     _ptr(C0) if have_state else None,
                                     _ptr(n0) if have_state else None,
                                     _ptr(m0) if have_state else None,
                                     _ptr(h), _ptr(C), _ptr(n), _ptr(m))
        if rc != 0:
            raise ValueError("oracle_fwd_f64 rejected its arguments")
        return h, C, n, m

    def step(self, q, k, v, i_pre, f_pre, o_pre, C, n, m):
        """One recurrent step.  q,k [B,NH,dqk], v,o_pre [B,NH,dv], i_pre,f_pre [B,NH].

        The state (C [B,NH,dv,dqk], n [B,NH,dqk], m [B,NH]) is copied, not modified.
        Returns (h [B,NH,dv], C, n, m) after the step.
        """
        q, k, v, i_pre, f_pre, o_pre = map(_f64, (q, k, v, i_pre, f_pre, o_pre))
        C, n, m = np.array(C, dtype=np.float64), np.array(n, dtype=np.float64), np.array(m, dtype=np.float64)
        B, NH, dqk = q.shape
        dv = v.shape[-1]
        assert C.shape == (B, NH, dv, dqk) and n.shape == (B, NH, dqk) and m.shape == (B, NH)
        h = np.empty((B, NH, dv))
        rc = self.lib.oracle_step_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre),
                                      B, NH, dqk, dv, _ptr(C), _ptr(n), _ptr(m), _ptr(h))
        if rc != 0:
            raise ValueError("oracle_step_f64 rejected its arguments")
        return h, C, n, m

    def bwd(self, q, k, v, i_pre, f_pre, o_pre, dh):
        """Gradients of the zero-state forward w.r.t. (q, k, v, i_pre, f_pre, o_pre) given dh.

        Shapes as fwd; dh like h.  Returns (dq, dk, dv, di, df, do) in fp64.
        """
        q, k, v, i_pre, f_pre, o_pre, dh = map(_f64, (q, k, v, i_pre, f_pre, o_pre, dh))
        B, NH, S, dqk = q.shape
        dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, NH, S, dv) and dh.shape == (B, NH, S, dv)
        assert i_pre.shape == (B, NH, S) and f_pre.shape == (B, NH, S) and o_pre.shape == (B, NH, S, dv)
        out = [np.empty_like(q), np.empty_like(k), np.empty_like(v), np.empty_like(i_pre),
               np.empty_like(f_pre), np.empty_like(o_pre)]
        rc = self.lib.oracle_bwd_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(o_pre), _ptr(dh),
                                     B, NH, S, dqk, dv, *[_ptr(a) for a in out])
        if rc != 0:
            raise ValueError("oracle_bwd_f64 rejected its arguments")
        return tuple(out)

    def epilogue(self, h, x, z, gn_w, gn_b, skip_w, eps, act):
        """mLSTM block epilogue: per-head GroupNorm of h, plus skip_w * x, gated by act(z).

        h, x, z [B,NH,S,dv]; gn_w, gn_b, skip_w [NH,dv]; act 0 = sigmoid, 1 = swish.
        Returns y [B,NH,S,dv] in fp64.
        """
        h, x, z, gn_w, gn_b, skip_w = map(_f64, (h, x, z, gn_w, gn_b, skip_w))
        B, NH, S, dv = h.shape
        assert x.shape == h.shape and z.shape == h.shape
        assert gn_w.shape == (NH, dv) and gn_b.shape == (NH, dv) and skip_w.shape == (NH, dv)
        y = np.empty_like(h)
        rc = self.lib.oracle_epilogue_f64(_ptr(h), _ptr(x), _ptr(z), _ptr(gn_w), _ptr(gn_b), _ptr(skip_w),
                                          B, NH, S, dv, float(eps), int(act), _ptr(y))
        if rc != 0:
            raise ValueError("oracle_epilogue_f64 rejected its arguments")
        return y

    def slstm(self, x_pre, R, forget_exp=0, c0=None, n0=None, m0=None, h0=None):
        """sLSTM recurrence.  x_pre [B,NH,S,4,dh] (gates z, i, f, o), R [NH,4,dh,dh].

        Returns (h [B,NH,S,dh], c, n, m, h_last [B,NH,dh]) in fp64; the state is the
        stabilized one.  All of c0, n0, m0, h0 None = zero state.
        """
        x_pre, R = _f64(x_pre), _f64(R)
        B, NH, S, four, dh = x_pre.shape
        assert four == 4 and R.shape == (NH, 4, dh, dh)
        st = [c0, n0, m0, h0]
        if any(a is not None for a in st):
            st = [_f64(a) for a in st]
            assert all(a.shape == (B, NH, dh) for a in st)
        h = np.empty((B, NH, S, dh))
        outs = [np.empty((B, NH, dh)) for _ in range(4)]
        rc = self.lib.oracle_slstm_f64(_ptr(x_pre), _ptr(R), B, NH, S, dh, int(forget_exp),
                                       *[_ptr(a) if a is not None else None for a in st],
                                       _ptr(h), *[_ptr(a) for a in outs])
        if rc != 0:
            raise ValueError("oracle_slstm_f64 rejected its arguments")
        return (h, *outs)

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())


def fwd(*args, **kwargs):
    return Oracle().fwd(*args, **kwargs)


def step(*args, **kwargs):
    return Oracle().step(*args, **kwargs)
