"""Calls enqueued on a stream other than torch's current one.

The binding allocates the workspace and any missing outputs with torch on the
current stream and hands their pointers to kernels enqueued on the caller's
stream.  The wrapper then drops the workspace while those kernels may still run;
the caching allocator must not give that memory to the next allocation on the
current stream before they finish.  Each test makes that next allocation at once
and writes over it, then checks the results against the oracle.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def test_forward_on_a_side_stream():
    import torch
    from mlstm_matrix_memory_amd import MLSTM_BF16, mlstm_fwd_parallel, mlstm_fwd_workspace_bytes
    w = inputs.WORKLOADS["lm_125m"]
    over = dict(B=2, NH=4, S=1024)
    announce(f"fwd on a side stream {over} d=384 chunk=64")
    x = inputs.fwd_inputs(w, seed=810, **over)
    dev = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    torch.cuda.synchronize()
    need = mlstm_fwd_workspace_bytes(2, 4, 1024, 384, 384, 64, MLSTM_BF16)
    assert need > 0
    side = torch.cuda.Stream()
    h, C, n, m = mlstm_fwd_parallel(*dev, 64, stream=side)
    # the next allocations on the current stream, written at once
    junk = [torch.full((need // 4 + 1024,), 7.0, dtype=torch.float32, device="cuda") for _ in range(4)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    rh, rC, rn, rm = oracle.Oracle().fwd(*(x[key] for key in KEYS))
    errs = {}
    for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
        check(name, to_np(g), r, TOL["bf16"], errs)


def test_step_on_a_side_stream():
    import torch
    from mlstm_matrix_memory_amd import mlstm_step
    w = inputs.WORKLOADS["decode"]
    B, NH, d = 16, 4, 512
    announce(f"mlstm_step on a side stream B={B} NH={NH} d={d}")
    st = inputs.step_state(w, seed=811, B=B, NH=NH, dqk=d, dv=d)
    xs = inputs.step_inputs(w, steps=1, seed=811, B=B, NH=NH, dqk=d, dv=d)
    C, n, m = (to_gpu(st[key], "f32") for key in ("C", "n", "m"))
    dev = [to_gpu(xs[key][0], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    h = mlstm_step(*dev, C, n, m, stream=side)
    junk = [torch.full((B * NH * d,), 3.0, dtype=torch.bfloat16, device="cuda") for _ in range(8)]
    side.synchronize()
    torch.cuda.synchronize()
    del junk
    rh, rC, rn, rm = oracle.Oracle().step(*(xs[key][0] for key in KEYS), st["C"], st["n"], st["m"])
    errs = {}
    for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
        check(name, to_np(g), r, TOL["bf16"], errs)
