"""GPU parity of the bf16 forward at key widths that are not multiples of 64.

The matrix-core forward has tilings for key widths that are multiples of 64 up
to 1024.  Other bf16 widths below 1024 run it on zero-padded copies of q and k
(and of a given C'_0, n'_0): q and k enter the cell only through contractions
over the key dimension ("xLSTM: Extended Long Short-Term Memory", section 2.3,
eq. (18) and the normalizer after it), so zero key columns leave every output
unchanged and the narrowed-back state is the unpadded one.  Each case is compared
element by element with the fp64 oracle on every output, and the staged entry
points with the whole call bit for bit.
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


# (chunk, d_qk, d_v): padded to 128, 64, 192, 128, 256, 512 (streaming scan) and
# 1024 (streaming scan), with partial value tiles
PADDED = [(64, 96, 80), (64, 48, 64), (32, 160, 48), (16, 80, 96), (128, 208, 144), (64, 464, 96),
          (64, 1008, 48), (64, 16, 32)]


@pytest.mark.parametrize("chunk,dqk,dv", PADDED, ids=lambda v: str(v))
def test_bf16_padded_key_widths(orc, chunk, dqk, dv):
    from mlstm_matrix_memory_amd import MLSTM_BF16, mlstm_fwd_workspace_bytes
    announce(f"fwd bf16 padded B=1 NH=2 S=256 dqk={dqk} dv={dv} chunk={chunk}")
    # the matrix-core path (the only one with a workspace) serves this width
    assert mlstm_fwd_workspace_bytes(1, 2, 256, dqk, dv, chunk, MLSTM_BF16) > 0
    x = inputs.fwd_inputs(inputs.WORKLOADS["lm_125m"], seed=900 + dqk + dv, B=1, NH=2, S=256, dqk=dqk, dv=dv)
    h, C, n, m = fwd_gpu(x, chunk, "bf16")
    rh, rC, rn, rm = orc.fwd(*(x[key] for key in KEYS))
    errs = {}
    for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
        check(name, g, r, TOL["bf16"], errs)


@pytest.mark.parametrize("over,cuts,chunk", [
    (dict(B=2, NH=1, S=300, dqk=96, dv=64), (100, 229), 64),     # padded MFMA parts, ragged tails, given states
    (dict(B=1, NH=1, S=200, dqk=1008, dv=64), (70,), 64),        # streaming scan from a padded state
], ids=lambda v: str(v))
def test_state_forward_in_pieces_padded(orc, over, cuts, chunk):
    import torch
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel_state
    announce(f"fwd_state bf16 padded {over} cuts={cuts} chunk={chunk}")
    x = inputs.fwd_inputs(inputs.WORKLOADS["lm_125m"], seed=950, **over)
    S = x["q"].shape[2]
    dev = {key: to_gpu(val, "bf16" if key in ("q", "k", "v") else "f32") for key, val in x.items()}
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
    check("h", np.concatenate(hs, axis=2), rh, TOL["bf16"], errs)
    check("C", to_np(state[0]), rC, TOL["bf16"], errs)
    check("n", to_np(state[1]), rn, TOL["bf16"], errs)
    check("m", to_np(state[2]), rm, TOL["bf16"], errs)


@pytest.mark.parametrize("dqk,dv", [(96, 80), (1008, 32)])
def test_staged_calls_equal_the_whole_call_padded(dqk, dv):
    import torch
    from mlstm_matrix_memory_amd import (MLSTM_BF16, mlstm_fwd_parallel, mlstm_fwd_prepare, mlstm_fwd_scan,
                                         mlstm_fwd_workspace_bytes)
    announce(f"fwd bf16 padded staged B=1 NH=2 S=256 dqk={dqk} dv={dv}")
    x = inputs.fwd_inputs(inputs.WORKLOADS["lm_125m"], seed=970, B=1, NH=2, S=256, dqk=dqk, dv=dv)
    args = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    whole = [t.clone() for t in mlstm_fwd_parallel(*args, 64)]
    need = mlstm_fwd_workspace_bytes(1, 2, 256, dqk, dv, 64, MLSTM_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    h = torch.empty_like(whole[0])
    C, n, m = (torch.empty_like(t) for t in whole[1:])
    mlstm_fwd_prepare(*args, 64, ws)
    mlstm_fwd_scan(*args, 64, h, C, n, m, ws)
    torch.cuda.synchronize()
    for name, a, b in zip("hCnm", whole, (h, C, n, m)):
        assert torch.equal(a, b), f"{name} differs between the staged and the whole call"
