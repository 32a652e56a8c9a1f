"""GPU parity of mlstm_fwd_parallel_block: the forward and the mLSTM block's
epilogue in one call, against the fp64 oracle's epilogue applied to the fp64
oracle's forward ("xLSTM: Extended Long Short-Term Memory", section 2.3 for the
cell, Figure 10 and its caption for the epilogue).

With fuse=1, shapes whose forward runs whole on the matrix cores with one
64-column value tile per head and one key part take the fused path (the scan
normalizes each row of h in registers); every other call runs the forward into
the workspace and the epilogue kernel after it.  Which path a call takes shows
in the workspace: the fused path needs exactly the forward's own.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _run(orc, over, chunk, dtype, act, fused, seed, fuse=1):
    import torch
    from mlstm_matrix_memory_amd import (MLSTM_BF16, MLSTM_F32, mlstm_fwd_block_workspace_bytes,
                                         mlstm_fwd_parallel_block, mlstm_fwd_workspace_bytes)
    w = inputs.WORKLOADS["lm_125m" if dtype == "bf16" else "tiny"]
    x = inputs.fwd_inputs(w, seed=seed, **over)
    B, NH, S, dqk = x["q"].shape
    dv = x["v"].shape[-1]
    e = inputs.epilogue_inputs(w, seed=seed, B=B, NH=NH, S=S, dv=dv)
    code = MLSTM_BF16 if dtype == "bf16" else MLSTM_F32
    own = mlstm_fwd_workspace_bytes(B, NH, S, dqk, dv, chunk, code)
    blk = mlstm_fwd_block_workspace_bytes(B, NH, S, dqk, dv, chunk, code, fuse)
    assert (blk == own) == fused, (own, blk)
    dev = [to_gpu(x[key], dtype if key in ("q", "k", "v") else "f32") for key in KEYS]
    xe, ze = to_gpu(e["x"], dtype), to_gpu(e["z"], dtype)
    gw, gb, sw = (to_gpu(e[n], "f32") for n in ("gn_w", "gn_b", "skip_w"))
    y, C, n, m = mlstm_fwd_parallel_block(*dev, xe, ze, gw, gb, sw, chunk, eps=1e-5, act=act, fuse=fuse)
    torch.cuda.synchronize()
    rh, rC, rn, rm = orc.fwd(*(x[key] for key in KEYS))
    ry = orc.epilogue(rh, e["x"], e["z"], e["gn_w"], e["gn_b"], e["skip_w"], 1e-5, act)
    errs = {}
    tol = TOL[dtype]
    check("y", to_np(y), ry, tol, errs)
    check("C", to_np(C), rC, tol, errs)
    check("n", to_np(n), rn, tol, errs)
    check("m", to_np(m), rm, tol, errs)
    return errs


FUSED = [
    # (overrides, chunk): one 64-column value tile per head
    (dict(B=2, NH=3, S=256, dqk=64, dv=64), 64),
    (dict(B=1, NH=2, S=256, dqk=128, dv=48), 64),        # partial tile: 48 of 64 columns
    (dict(B=2, NH=1, S=256, dqk=96, dv=32), 64),         # key width padded to 128, half a tile
    (dict(B=1, NH=2, S=256, dqk=64, dv=64), 16),         # 16-token chunks run as 64-token ones
    (dict(B=1, NH=2, S=256, dqk=128, dv=64), 32),        # the 32-token tiling of width 128
    (dict(B=1, NH=1, S=4096, dqk=128, dv=64), 64),       # several sequence segments
    (dict(B=1, NH=2, S=2048, dqk=64, dv=64), 64),        # segments at width 64
]


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("over,chunk", FUSED, ids=lambda v: str(v))
def test_fused(orc, over, chunk, act):
    announce(f"fwd+epilogue fused {over} chunk={chunk} act={act}")
    _run(orc, over, chunk, "bf16", act, True, seed=1200 + over["dqk"] + over["dv"])


UNFUSED = [
    # (overrides, chunk, dtype)
    (dict(B=1, NH=2, S=256, dqk=384, dv=384), 64, "bf16"),    # several value tiles per head
    (dict(B=1, NH=2, S=512, dqk=384, dv=64), 64, "bf16"),     # one tile, but two key parts per tile
    (dict(B=1, NH=1, S=256, dqk=1024, dv=64), 64, "bf16"),    # the streaming form of the scan
    (dict(B=1, NH=2, S=256, dqk=2048, dv=32), 64, "bf16"),    # the vector-ALU forward
    (dict(B=2, NH=2, S=128, dqk=48, dv=80), 16, "f32"),       # the fp32 path
]


@pytest.mark.parametrize("over,chunk,dtype", UNFUSED, ids=lambda v: str(v))
def test_unfused(orc, over, chunk, dtype):
    # fuse=1 asked for, but these shapes have no fusable tiling
    announce(f"fwd+epilogue unfused {over} chunk={chunk} {dtype}")
    _run(orc, over, chunk, dtype, 1, False, seed=1300 + over["dqk"] + over["dv"])


@pytest.mark.parametrize("over,chunk", FUSED[:2], ids=lambda v: str(v))
def test_fuse_zero_runs_two_passes(orc, over, chunk):
    announce(f"fwd+epilogue fuse=0 {over} chunk={chunk}")
    _run(orc, over, chunk, "bf16", 0, False, seed=1500 + over["dqk"], fuse=0)


def test_fused_equals_forward_then_epilogue_up_to_rounding():
    # the fused path normalizes h before rounding it; the two-call path rounds h to
    # bf16 first, so they agree to the bf16 rounding of h
    import torch
    from mlstm_matrix_memory_amd import mlstm_block_epilogue, mlstm_fwd_parallel, mlstm_fwd_parallel_block
    announce("fwd+epilogue fused against mlstm_fwd_parallel then mlstm_block_epilogue, B=2 NH=4 S=512 d=64")
    w = inputs.WORKLOADS["lm_125m"]
    x = inputs.fwd_inputs(w, seed=1400, B=2, NH=4, S=512, dqk=64, dv=64)
    e = inputs.epilogue_inputs(w, seed=1400, B=2, NH=4, S=512, dv=64)
    dev = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    xe, ze = to_gpu(e["x"], "bf16"), to_gpu(e["z"], "bf16")
    gw, gb, sw = (to_gpu(e[n], "f32") for n in ("gn_w", "gn_b", "skip_w"))
    y, C, n, m = mlstm_fwd_parallel_block(*dev, xe, ze, gw, gb, sw, 64, eps=1e-5, act=1, fuse=1)
    h, C2, n2, m2 = mlstm_fwd_parallel(*dev, 64)
    y2 = mlstm_block_epilogue(h, xe, ze, gw, gb, sw, eps=1e-5, act=1)
    torch.cuda.synchronize()
    assert torch.equal(C, C2) and torch.equal(n, n2) and torch.equal(m, m2)
    errs = {}
    check("y", to_np(y), to_np(y2), 2e-2, errs)


# (batch index, head index) of the sampled heads
SAMPLED = [(0, 0), (3, 7), (7, 15)]


@pytest.mark.parametrize("fuse", [1, 0])
def test_full_size_heads64_sampled_heads(orc, fuse):
    """The whole 16-head workload (B=8, NH=16, S=2048, d=64, chunk 64) in the launch
    configuration the benchmark times, compared with the oracle on sampled heads
    (each head is an independent recurrence and its own GroupNorm group)."""
    import torch
    from mlstm_matrix_memory_amd import (MLSTM_BF16, mlstm_fwd_block_workspace_bytes, mlstm_fwd_parallel_block,
                                         mlstm_fwd_workspace_bytes)
    w = inputs.WORKLOADS["heads64"]
    announce(f"fwd+epilogue full size heads64 B={w.B} NH={w.NH} S={w.S} d={w.dqk} fuse={fuse}")
    own = mlstm_fwd_workspace_bytes(w.B, w.NH, w.S, w.dqk, w.dv, w.chunk, MLSTM_BF16)
    assert (mlstm_fwd_block_workspace_bytes(w.B, w.NH, w.S, w.dqk, w.dv, w.chunk, MLSTM_BF16, fuse) == own) == bool(fuse)
    x = inputs.fwd_inputs(w)
    e = inputs.epilogue_inputs(w)
    dev = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    xe, ze = to_gpu(e["x"], "bf16"), to_gpu(e["z"], "bf16")
    gw, gb, sw = (to_gpu(e[n], "f32") for n in ("gn_w", "gn_b", "skip_w"))
    y, C, n, m = mlstm_fwd_parallel_block(*dev, xe, ze, gw, gb, sw, w.chunk, eps=1e-5, act=1, fuse=fuse)
    torch.cuda.synchronize()
    y, C, n, m = to_np(y), to_np(C), to_np(n), to_np(m)
    errs = {}
    for b, h in SAMPLED:
        one = {key: x[key][b:b + 1, h:h + 1] for key in KEYS}
        rh, rC, rn, rm = orc.fwd(*(one[key] for key in KEYS))
        ry = orc.epilogue(rh, e["x"][b:b + 1, h:h + 1], e["z"][b:b + 1, h:h + 1], e["gn_w"][h:h + 1],
                          e["gn_b"][h:h + 1], e["skip_w"][h:h + 1], 1e-5, 1)
        check(f"y{b},{h}", y[b:b + 1, h:h + 1], ry, TOL["bf16"], errs)
        check(f"C{b},{h}", C[b:b + 1, h:h + 1], rC, TOL["bf16"], errs)
        check(f"n{b},{h}", n[b:b + 1, h:h + 1], rn, TOL["bf16"], errs)
        check(f"m{b},{h}", m[b:b + 1, h:h + 1], rm, TOL["bf16"], errs)
    assert np.all(np.isfinite(y))
    print(errs)
