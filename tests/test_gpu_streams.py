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


def test_library_loaded_before_torch_touches_the_gpu():
    # A fresh process that loads the library (a workspace query) before torch has
    # used the GPU must still launch on torch's HIP runtime: the binding imports
    # torch before loading the library, so one runtime serves both.
    import os
    import subprocess
    import sys
    announce("fwd in a fresh process that loads the library before torch uses the GPU")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from mlstm_matrix_memory_amd import MLSTM_BF16, mlstm_fwd_workspace_bytes, mlstm_fwd_parallel\n"
        "assert mlstm_fwd_workspace_bytes(1, 2, 128, 96, 64, 64, MLSTM_BF16) > 0\n"
        "import torch\n"
        "g = torch.Generator().manual_seed(1)\n"
        "q, k = (torch.randn(1, 2, 128, 96, generator=g).to('cuda', torch.bfloat16) for _ in range(2))\n"
        "v = torch.randn(1, 2, 128, 64, generator=g).to('cuda', torch.bfloat16)\n"
        "i, f = (torch.randn(1, 2, 128, generator=g).cuda() for _ in range(2))\n"
        "o = torch.randn(1, 2, 128, 64, generator=g).cuda()\n"
        "h, C, n, m = mlstm_fwd_parallel(q, k, v, i, f + 3.0, o, 64)\n"
        "torch.cuda.synchronize()\n"
        "assert bool(torch.isfinite(h.float()).all()) and bool(torch.isfinite(C).all())\n"
        "print('ok')\n" % root)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
