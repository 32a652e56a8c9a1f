"""GPU parity of mlstm_fwd_parallel_state: a forward that continues from a given
stabilized state and accepts any sequence length.

A sequence run in pieces -- each piece from the state the previous piece
returned, piece lengths not multiples of the chunk -- must give the oracle's
result for one run over the whole sequence ("xLSTM: Extended Long Short-Term
Memory", section 2.3: the state carried across the chunks of the parallel form).
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

KEYS = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def _pieces(orc, w, dtype, over, cuts, chunk, seed, f_shift=0.0):
    import torch
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel_state
    x = inputs.fwd_inputs(w, seed=seed, **over)
    x["f_pre"] = x["f_pre"] + np.float32(f_shift)
    S = x["q"].shape[2]
    dev = {key: to_gpu(val, dtype if key in ("q", "k", "v") else "f32") for key, val in x.items()}
    bounds = [0] + list(cuts) + [S]
    hs, state = [], (None, None, None)
    for a, b in zip(bounds[:-1], bounds[1:]):
        piece = [dev[key][:, :, a:b].contiguous() for key in KEYS]
        h, C, n, m = mlstm_fwd_parallel_state(*piece, chunk, *state)
        hs.append(to_np(h))
        state = (C.clone(), n.clone(), m.clone())      # the next piece may not share the buffers
    torch.cuda.synchronize()
    rh, rC, rn, rm = orc.fwd(*(x[key] for key in KEYS))
    errs = {}
    tol = TOL[dtype]
    check("h", np.concatenate(hs, axis=2), rh, tol, errs)
    check("C", to_np(state[0]), rC, tol, errs)
    check("n", to_np(state[1]), rn, tol, errs)
    check("m", to_np(state[2]), rm, tol, errs)
    return errs


CASES = [
    # (workload, overrides, cuts, chunk, dtype): cuts split the sequence into pieces
    ("lm_125m", dict(B=1, NH=2, S=700), (512,), 64, "bf16"),          # MFMA part + ragged tail
    ("lm_125m", dict(B=2, NH=1, S=333, dqk=128, dv=96), (100, 260), 32, "bf16"),  # every piece ragged
    ("lm_1_3b", dict(B=1, NH=1, S=300), (64,), 64, "bf16"),
    ("lm_1_3b", dict(B=1, NH=2, S=1100, dqk=512, dv=512), (320,), 64, "bf16"),   # streaming scan from a state
    ("long_ctx", dict(B=1, NH=1, S=3000, dqk=256, dv=256), (1024,), 64, "bf16"),  # segments from a state
    ("lm_125m", dict(B=1, NH=2, S=3000, dqk=64, dv=64), (1024,), 64, "bf16"),      # segments from a state, d 64
    ("long_ctx", dict(B=1, NH=2, S=1100), (129,), 128, "bf16"),
    ("tiny", dict(B=2, NH=2, S=150, dqk=48, dv=80), (37, 100), 16, "f32"),
]


@pytest.mark.parametrize("name,over,cuts,chunk,dtype", CASES, ids=lambda v: str(v))
def test_pieces_continue_the_sequence(orc, name, over, cuts, chunk, dtype):
    w = inputs.WORKLOADS[name]
    announce(f"fwd_state pieces {name} {over} cuts={cuts} chunk={chunk} {dtype}")
    errs = _pieces(orc, w, dtype, over, cuts, chunk, seed=500 + w.seed)
    print(name, errs)


def test_segments_from_a_state_under_slow_decay(orc):
    # Forget gates close to one (f~ ~ N(8, 1)), so the state handed between pieces and
    # every token part of every segment reach the later outputs.  With 8 heads of
    # width 256 the second piece (2048 tokens through the MFMA path, then a ragged
    # tail of 52) runs as 4 segments of 2 token parts each, from the first piece's state.
    w = inputs.WORKLOADS["lm_125m"]
    over = dict(B=1, NH=8, S=4100, dqk=256, dv=256)
    announce(f"fwd_state pieces slow decay {over} cuts=(2000,) chunk=64 bf16")
    errs = _pieces(orc, w, "bf16", over, (2000,), 64, seed=530, f_shift=5.0)
    print(errs)


def test_state_forward_from_zero_equals_the_plain_forward():
    import torch
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel, mlstm_fwd_parallel_state
    w = inputs.WORKLOADS["lm_125m"]
    announce("fwd_state zero state vs fwd_parallel B=1 NH=2 S=512 d=384")
    x = inputs.fwd_inputs(w, seed=9, B=1, NH=2, S=512)
    dev = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    a = mlstm_fwd_parallel(*dev, 64)
    b = mlstm_fwd_parallel_state(*dev, 64)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert np.array_equal(to_np(u), to_np(v))
