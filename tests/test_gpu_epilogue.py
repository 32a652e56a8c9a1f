"""GPU parity of mlstm_block_epilogue against the fp64 oracle's epilogue.

The epilogue is one pass per (batch, head, token) row, so the oracle covers every
element even at the full lm_125m and lm_1_3b sizes.
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _run(e, dtype, eps, act, inplace=None):
    import torch
    from mlstm_matrix_memory_amd import mlstm_block_epilogue
    h, x, z = (to_gpu(e[n], dtype) for n in ("h", "x", "z"))
    gw, gb, sw = (to_gpu(e[n], "f32") for n in ("gn_w", "gn_b", "skip_w"))
    out = {"h": h, "x": x, "z": z}.get(inplace)
    y = mlstm_block_epilogue(h, x, z, gw, gb, sw, eps=eps, act=act, y_out=out)
    torch.cuda.synchronize()
    return to_np(y)


def _compare(orc, e, dtype, eps=1e-5, act=0, inplace=None):
    y = _run(e, dtype, eps, act, inplace)
    r = orc.epilogue(e["h"], e["x"], e["z"], e["gn_w"], e["gn_b"], e["skip_w"], eps, act)
    errs = {}
    # against the oracle itself, and (bf16) against its output rounded as y is stored
    check("y", y, r, TOL[dtype], errs)
    if dtype == "bf16":
        check("y_rounded", y, inputs.bf16_round(r.astype(np.float32)).astype(np.float64), TOL[dtype], errs)
    return errs


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("dv", [16, 48, 256, 272, 1024, 4096])
def test_fp32_widths(orc, dv, act):
    w = inputs.WORKLOADS["tiny"]
    announce(f"epilogue fp32 B=2 NH=3 S=37 dv={dv} act={act}")
    _compare(orc, inputs.epilogue_inputs(w, seed=500 + dv, B=2, NH=3, S=37, dv=dv), "f32", act=act)


@pytest.mark.parametrize("act", [0, 1])
@pytest.mark.parametrize("name", ["lm_125m", "lm_1_3b"])
def test_bf16_full_size(orc, name, act):
    w = inputs.WORKLOADS[name]
    announce(f"epilogue bf16 {name} full size act={act}")
    _compare(orc, inputs.epilogue_inputs(w), "bf16", act=act)


@pytest.mark.parametrize("which", ["h", "x", "z"])
def test_in_place(orc, which):
    w = inputs.WORKLOADS["lm_125m"]
    announce(f"epilogue bf16 in place over {which}")
    _compare(orc, inputs.epilogue_inputs(w, seed=510, B=1, NH=4, S=64), "bf16", act=1, inplace=which)


def test_constant_rows_need_eps(orc):
    # rows with one value everywhere normalize to 0: y = (gn_b + skip_w x) act(z)
    w = inputs.WORKLOADS["tiny"]
    announce("epilogue fp32 constant rows")
    e = inputs.epilogue_inputs(w, seed=520, B=1, NH=2, S=9, dv=32)
    e["h"][:] = e["h"][..., :1]
    _compare(orc, e, "f32", eps=1e-3)


def test_after_forward(orc):
    # the epilogue applied to the h the GPU forward produced (both sides get that h)
    import torch
    from gpu_helpers import fwd_gpu
    w = inputs.WORKLOADS["lm_125m"]
    announce("epilogue bf16 after mlstm_fwd_parallel B=1 NH=4 S=256")
    x = inputs.fwd_inputs(w, seed=530, B=1, NH=4, S=256)
    h = fwd_gpu(x, 64, "bf16")[0]
    e = inputs.epilogue_inputs(w, seed=530, B=1, NH=4, S=256)
    e["h"] = h.astype(np.float32)
    _compare(orc, e, "bf16", act=1)
