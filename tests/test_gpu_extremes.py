"""GPU parity in the gate regimes the oracle is pinned on.

"xLSTM: Extended Long Short-Term Memory", section 2.2 (eq. (17) and the sentence
after it: the stabilizer keeps exponential input gates finite and changes no
output) and section 2.3 (eq. (18), the covariance update, and the normalizer
with its floor).  These inputs reach the paths ordinary draws do not:

* extreme finite gates -- f~ = -750 (sigmoid underflows, log sigmoid is exactly
  -750), f~ = +750, f~ = -60, input-gate spikes i~ = 40 and a closed input gate
  i~ = -300 -- which drive the in-chunk cumulative sums to about -750 per token,
  the carried decay of a chunk to exactly zero in fp32 (the lazy rescale of the
  state registers), and the floor exp(-m) below the fp32 range;
* input-gate spikes i~ = 800 and 720 followed by deep forgets f~ = -750 and -715,
  placed mid-chunk, across a chunk boundary and across a sequence-segment
  boundary: after them the memory is one stored pair, and queries nearly
  orthogonal to its key retrieve a strongly cancelling C'q;
* f~ = +30 with i~ = 0: no decay and unit input gates, the plain accumulation of
  eq. (18) (C' = V^T K, m = 0);
* f~ = -30: the memoryless case, each token sees only itself.

Every case is compared element by element with the oracle on every output (h,
C', n', m), at 2e-2 for bf16 inputs and 1e-4 for the fp32 path.  The same gate
extremes go through mlstm_fwd_parallel_state (pieces of 1 and 17 tokens, a
one-token piece between two longer ones) and through mlstm_step.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, fwd_gpu, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _pattern(x, name, L, seg=None):
    """Apply one gate pattern to copies of the inputs (all heads alike)."""
    y = {key: val.copy() for key, val in x.items()}
    i, f = y["i_pre"], y["f_pre"]
    S = i.shape[-1]
    if name == "extreme":
        f[..., L // 2 + 5] = -750.0
        f[..., 3 * L // 2 + 9] = 750.0
        f[..., min(S - 1, 2 * L + 20)] = -60.0
        i[..., 3] = 40.0
        i[..., L + 17] = 40.0
        i[..., min(S - 1, 2 * L + 2)] = -300.0
    elif name == "spike_forget":
        i[..., 10] = 800.0                     # mid-chunk
        f[..., 11] = -750.0
        tb = 3 * L - 1 if 3 * L < S else L - 1  # last token of a chunk, forget on the next one's first
        i[..., tb] = 720.0
        f[..., tb + 1] = -715.0
        if seg is not None and seg < S:        # across a sequence-segment boundary
            i[..., seg - 1] = 800.0
            f[..., seg] = -750.0
        i[..., S - L] = 800.0                  # on the first token of the last chunk, no forget after it
    elif name == "eq18":
        f[...] = 30.0
        i[...] = 0.0
    elif name == "memoryless":
        f[...] = -30.0
    else:
        raise ValueError(name)
    return y


def _compare(orc, x, chunk, dtype):
    h, C, n, m = fwd_gpu(x, chunk, dtype)
    for name, a in (("h", h), ("C", C), ("n", n), ("m", m)):
        assert np.all(np.isfinite(a)), f"{name} is not finite"
    rh, rC, rn, rm = orc.fwd(*(x[key] for key in KEYS))
    errs = {}
    for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
        check(name, g, r, TOL[dtype], errs)
    return errs


PATTERNS = ["extreme", "spike_forget", "eq18", "memoryless"]

# (label, workload, overrides, chunk, dtype, tokens per sequence segment of the scan)
SHAPES = [
    # the bf16 MFMA tiling of width 384 (8 chunks, 6 value tiles per head)
    ("mfma_d384", "lm_125m", dict(B=1, NH=2, S=512), 64, "bf16", None),
    # the bf16 MFMA tiling of width 1024
    ("mfma_d1024", "lm_1_3b", dict(B=1, NH=1, S=256), 64, "bf16", None),
    # one head of width 256 over 4096 tokens: the scan runs it as 8 sequence
    # segments of 512 tokens, each from its own entering state
    ("segmented", "long_ctx", dict(B=1, NH=1, S=4096, dqk=256, dv=256), 128, "bf16", 512),
    # width 512 (the streaming form of the scan) over 2048 tokens: 8 segments of 256
    ("streaming_segmented", "lm_1_3b", dict(B=1, NH=1, S=2048, dqk=512, dv=512), 64, "bf16", 256),
    # a key width off the 64-column grid: zero-padded to the width-128 tiling
    ("padded_d96", "lm_125m", dict(B=1, NH=2, S=512, dqk=96, dv=80), 64, "bf16", None),
    # the fp32 path
    ("fp32_c64", "tiny", dict(B=1, NH=2, S=256, dqk=48, dv=80), 64, "f32", None),
    ("fp32_c16", "tiny", dict(B=1, NH=2, S=256, dqk=48, dv=80), 16, "f32", None),
]


@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("label,name,over,chunk,dtype,seg", SHAPES, ids=[s[0] for s in SHAPES])
def test_fwd_gate_regimes(orc, label, name, over, chunk, dtype, seg, pattern):
    w = inputs.WORKLOADS[name]
    announce(f"fwd gate regime {pattern} {label} {over} chunk={chunk} {dtype}")
    x = inputs.fwd_inputs(w, seed=700 + len(label), **over)
    errs = _compare(orc, _pattern(x, pattern, 64 if chunk > 64 else chunk, seg), chunk, dtype)
    print(label, pattern, errs)


# ---------------------------------------------------------------------------
# mlstm_fwd_parallel_state: short pieces, each from the previous piece's state
# ---------------------------------------------------------------------------

def _pieces(orc, x, cuts, chunk, dtype):
    import torch
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel_state
    S = x["q"].shape[2]
    dev = {key: to_gpu(val, dtype if key in ("q", "k", "v") else "f32") for key, val in x.items()}
    bounds = [0] + list(cuts) + [S]
    hs, state = [], (None, None, None)
    for a, b in zip(bounds[:-1], bounds[1:]):
        piece = [dev[key][:, :, a:b].contiguous() for key in KEYS]
        h, C, n, m = mlstm_fwd_parallel_state(*piece, chunk, *state)
        hs.append(to_np(h))
        state = (C.clone(), n.clone(), m.clone())
    torch.cuda.synchronize()
    rh, rC, rn, rm = orc.fwd(*(x[key] for key in KEYS))
    errs = {}
    tol = TOL[dtype]
    check("h", np.concatenate(hs, axis=2), rh, tol, errs)
    check("C", to_np(state[0]), rC, tol, errs)
    check("n", to_np(state[1]), rn, tol, errs)
    check("m", to_np(state[2]), rm, tol, errs)
    return errs


STATE_CASES = [
    # (label, workload, overrides, cuts, chunk, dtype)
    ("S1_first", "lm_125m", dict(B=1, NH=2, S=200, dqk=384, dv=384), (1,), 64, "bf16"),
    ("S17_first", "lm_125m", dict(B=1, NH=2, S=200, dqk=384, dv=384), (17,), 64, "bf16"),
    ("one_token_between", "lm_125m", dict(B=1, NH=2, S=300, dqk=384, dv=384), (128, 129), 64, "bf16"),
    ("S1_only", "lm_125m", dict(B=2, NH=2, S=1, dqk=128, dv=96), (), 64, "bf16"),
    ("S17_only", "lm_1_3b", dict(B=1, NH=1, S=17), (), 64, "bf16"),
    ("padded_pieces", "lm_125m", dict(B=1, NH=2, S=200, dqk=96, dv=64), (1, 65), 64, "bf16"),
    ("fp32_short_pieces", "tiny", dict(B=2, NH=2, S=90, dqk=48, dv=80), (1, 18, 19), 16, "f32"),
]


@pytest.mark.parametrize("pattern", [None, "extreme", "spike_forget"])
@pytest.mark.parametrize("label,name,over,cuts,chunk,dtype", STATE_CASES, ids=[c[0] for c in STATE_CASES])
def test_state_forward_short_pieces(orc, label, name, over, cuts, chunk, dtype, pattern):
    w = inputs.WORKLOADS[name]
    announce(f"fwd_state {label} {over} cuts={cuts} chunk={chunk} {dtype} gates={pattern}")
    x = inputs.fwd_inputs(w, seed=740 + len(label), **over)
    S = over["S"]
    if pattern == "extreme" and S >= 200:
        x = _pattern(x, "extreme", 64)
    elif pattern == "spike_forget" and S >= 200:
        x = _pattern(x, "spike_forget", 64)
    elif pattern is not None:
        # short sequences: a spike on the first token, a deep forget on the next, a closed input gate
        x["i_pre"][..., 0] = 800.0
        if S > 1:
            x["f_pre"][..., 1] = -750.0
        if S > 3:
            x["i_pre"][..., 3] = -300.0
            x["f_pre"][..., S - 1] = 750.0
    errs = _pieces(orc, x, cuts, chunk, dtype)
    print(label, pattern, errs)


# ---------------------------------------------------------------------------
# mlstm_step under the same gate extremes
# ---------------------------------------------------------------------------

# per step: (i~, f~) overrides for every head; None keeps the drawn value
STEP_GATES = [(800.0, None), (None, -750.0), (0.0, 30.0), (None, -30.0), (720.0, None), (None, -715.0),
              (None, 750.0), (-300.0, None), (40.0, -60.0), (None, None)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dqk,dv", [(64, 48), (512, 512)])
def test_step_gate_extremes(orc, dtype, dqk, dv):
    """Each step against the oracle's step from the state the kernel was given.

    mlstm_step maps an fp32 state to an fp32 state, so its reference is the oracle's
    step applied to that same state (exactly upcast).  After a spike the memory is
    one stored pair; a query nearly orthogonal to its key then makes h a ratio of
    two strongly cancelling dot products, and the fp32 rounding of the stored state
    itself (which any fp32 state carries) is amplified accordingly.  Chaining the
    steps against the oracle's fp64 chain would charge that storage rounding to
    the kernel; for bf16 inputs the chain is compared as well, at its tolerance.
    """
    import dataclasses
    import torch
    from mlstm_matrix_memory_amd import mlstm_step
    w = dataclasses.replace(inputs.WORKLOADS["decode"], dtype=dtype)
    B, NH, T = 3, 2, len(STEP_GATES)
    announce(f"mlstm_step gate extremes {dtype} B={B} NH={NH} dqk={dqk} dv={dv} steps={T}")
    st = inputs.step_state(w, seed=760, B=B, NH=NH, dqk=dqk, dv=dv)
    xs = inputs.step_inputs(w, steps=T, seed=760, B=B, NH=NH, dqk=dqk, dv=dv)
    for t, (gi, gf) in enumerate(STEP_GATES):
        if gi is not None:
            xs["i_pre"][t] = gi
        if gf is not None:
            xs["f_pre"][t] = gf
    C, n, m = (to_gpu(st[key], "f32") for key in ("C", "n", "m"))
    dev = {key: to_gpu(xs[key], dtype if key in ("q", "k", "v") else "f32") for key in xs}
    errs = {}
    cC, cn, cm = st["C"], st["n"], st["m"]        # the oracle's own fp64 chain
    for t in range(T):
        given = (to_np(C), to_np(n), to_np(m))
        h = mlstm_step(*(dev[key][t] for key in KEYS), C, n, m)
        torch.cuda.synchronize()
        rh, rC, rn, rm = orc.step(*(xs[key][t] for key in KEYS), *given)
        for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
            check(f"{name} step {t}", to_np(g), r, TOL[dtype], errs)
        ch, cC, cn, cm = orc.step(*(xs[key][t] for key in KEYS), cC, cn, cm)
        if dtype == "bf16":
            check(f"h step {t} (chain)", to_np(h), ch, TOL[dtype], errs)
    if dtype == "bf16":
        check("C (chain)", to_np(C), cC, TOL[dtype], errs)
        check("n (chain)", to_np(n), cn, TOL[dtype], errs)
        check("m (chain)", to_np(m), cm, TOL[dtype], errs)
    print(errs)
