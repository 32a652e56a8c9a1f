"""GPU parity of mlstm_step (one-token decode) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _run_steps(orc, w, steps, dtype, B, NH, dqk, dv, seed, sample_heads=None):
    import torch
    from mlstm_matrix_memory_amd import mlstm_step
    announce(f"mlstm_step {dtype} B={B} NH={NH} dqk={dqk} dv={dv} steps={steps} seed={seed}")
    st = inputs.step_state(w, seed=seed, B=B, NH=NH, dqk=dqk, dv=dv)
    xs = inputs.step_inputs(w, steps=steps, seed=seed, B=B, NH=NH, dqk=dqk, dv=dv)
    C = to_gpu(st["C"], "f32")
    n = to_gpu(st["n"], "f32")
    m = to_gpu(st["m"], "f32")
    dev_in = {key: to_gpu(xs[key], dtype if key in ("q", "k", "v") else "f32") for key in xs}
    hs = []
    for t in range(steps):
        h = mlstm_step(dev_in["q"][t], dev_in["k"][t], dev_in["v"][t], dev_in["i_pre"][t],
                       dev_in["f_pre"][t], dev_in["o_pre"][t], C, n, m)
        hs.append(h)
    torch.cuda.synchronize()
    h_gpu = np.stack([to_np(h) for h in hs])
    C_gpu, n_gpu, m_gpu = to_np(C), to_np(n), to_np(m)
    # every head, sampled by the oracle or not, stays finite through all the steps
    for name, a in (("h", h_gpu), ("C", C_gpu), ("n", n_gpu), ("m", m_gpu)):
        assert np.all(np.isfinite(a)), f"{name} is not finite"
    # oracle, optionally on a subset of heads
    if sample_heads is None:
        sel = (slice(None), slice(None))
    else:
        sel = sample_heads
    oC, on, om = st["C"][sel], st["n"][sel], st["m"][sel]
    ref_h = []
    for t in range(steps):
        hh, oC, on, om = orc.step(xs["q"][t][sel], xs["k"][t][sel], xs["v"][t][sel], xs["i_pre"][t][sel],
                                  xs["f_pre"][t][sel], xs["o_pre"][t][sel], oC, on, om)
        ref_h.append(hh)
    ref_h = np.stack(ref_h)
    return (h_gpu[(slice(None),) + sel], C_gpu[sel], n_gpu[sel], m_gpu[sel]), (ref_h, oC, on, om)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dqk,dv", [(64, 48), (16, 16), (272, 80), (1040, 32), (4096, 16), (32, 4096)])
def test_step_shapes(orc, dtype, dqk, dv):
    w = inputs.WORKLOADS["decode"]
    w = dataclasses.replace(w, dtype=dtype)
    got, ref = _run_steps(orc, w, 4, dtype, 3, 2, dqk, dv, seed=7)
    errs = {}
    for name, g, r in zip(("h", "C", "n", "m"), got, ref):
        check(name, g, r, TOL[dtype], errs)


def test_step_decode_workload(orc):
    """Full decode workload (batch 256, NH 4, d 512, 128 steps); oracle on sampled heads."""
    w = inputs.WORKLOADS["decode"]
    heads_b = np.array([[0, 17, 101, 255]])   # [1, n]: keeps the [B, NH] axes
    heads_h = np.array([[0, 3, 1, 2]])
    sel = (heads_b, heads_h)
    got, ref = _run_steps(orc, w, w.S, "bf16", w.B, w.NH, w.dqk, w.dv, seed=w.seed, sample_heads=sel)
    errs = {}
    for name, g, r in zip(("h", "C", "n", "m"), got, ref):
        check(name, g, r, TOL["bf16"], errs)
    print("decode errors", errs)


def test_step_is_deterministic():
    import torch
    from mlstm_matrix_memory_amd import mlstm_step
    announce("mlstm_step determinism B=8 NH=2 d=256")
    w = inputs.WORKLOADS["decode"]
    st = inputs.step_state(w, B=8, NH=2, dqk=256, dv=256)
    xs = inputs.step_inputs(w, steps=1, B=8, NH=2, dqk=256, dv=256)
    outs = []
    for _ in range(2):
        C, n, m = (to_gpu(st[key], "f32") for key in ("C", "n", "m"))
        d = {key: to_gpu(xs[key][0], "bf16" if key in "qkv" else "f32") for key in xs}
        h = mlstm_step(d["q"], d["k"], d["v"], d["i_pre"], d["f_pre"], d["o_pre"], C, n, m)
        torch.cuda.synchronize()
        outs.append([to_np(t) for t in (h, C, n, m)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
