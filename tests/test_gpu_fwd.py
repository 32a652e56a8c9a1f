"""GPU parity of mlstm_fwd_parallel against the fp64 oracle.

Sizes the oracle finishes in seconds (several tiles, ragged value tiles, every
chunk size) are compared element by element on every output; the full workload
sizes are run whole on the GPU in the benchmark's launch configuration and
compared on sampled heads (each head is an independent recurrence, so the
oracle computes exactly those heads' outputs).
"""
import numpy as np
import pytest

import oracle
from gpu_helpers import TOL, announce, check, fwd_gpu
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


def _compare(orc, x, chunk, dtype, sel=None):
    h, C, n, m = fwd_gpu(x, chunk, dtype)
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(C)) and np.all(np.isfinite(n)) and np.all(np.isfinite(m))
    if sel is not None:
        x = {key: val[sel] for key, val in x.items()}
        h, C, n, m = h[sel], C[sel], n[sel], m[sel]
    rh, rC, rn, rm = orc.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    errs = {}
    for name, g, r in (("h", h, rh), ("C", C, rC), ("n", n, rn), ("m", m, rm)):
        check(name, g, r, TOL[dtype], errs)
    return errs


@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_tiny_fp32(orc, chunk):
    w = inputs.WORKLOADS["tiny"]
    announce(f"fwd tiny fp32 chunk={chunk}")
    _compare(orc, inputs.fwd_inputs(w), chunk, "f32")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
@pytest.mark.parametrize("dqk,dv", [(48, 80), (16, 16), (128, 32)])
def test_fp32_medium(orc, chunk, dqk, dv):
    w = inputs.WORKLOADS["tiny"]
    announce(f"fwd fp32 B=2 NH=2 S=256 dqk={dqk} dv={dv} chunk={chunk}")
    x = inputs.fwd_inputs(w, seed=101, B=2, NH=2, S=256, dqk=dqk, dv=dv)
    _compare(orc, x, chunk, "f32")


REDUCED = [
    # (workload, overrides, chunk)
    ("lm_125m", dict(B=1, NH=2, S=512), 64),
    ("lm_125m", dict(B=2, NH=1, S=256, dqk=96, dv=48), 32),
    ("lm_1_3b", dict(B=1, NH=1, S=256), 64),
    ("long_ctx", dict(B=1, NH=2, S=2048), 128),
    ("long_ctx", dict(B=1, NH=1, S=512, dqk=64, dv=160), 16),
]


@pytest.mark.parametrize("name,over,chunk", REDUCED, ids=lambda v: str(v))
def test_bf16_reduced(orc, name, over, chunk):
    w = inputs.WORKLOADS[name]
    announce(f"fwd bf16 {name} {over} chunk={chunk}")
    x = inputs.fwd_inputs(w, seed=100 + w.seed, **over)
    _compare(orc, x, chunk, "bf16")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_bf16_chunk_sweep(orc, chunk):
    w = inputs.WORKLOADS["lm_125m"]
    announce(f"fwd bf16 chunk sweep B=1 NH=2 S=256 d=128 chunk={chunk}")
    x = inputs.fwd_inputs(w, seed=55, B=1, NH=2, S=256, dqk=128, dv=128)
    _compare(orc, x, chunk, "bf16")


# every (chunk, d_qk) the bf16 MFMA path has a tiling for, each with a d_v that
# leaves a partial value tile (d_v not a multiple of the tile width)
MFMA_SHAPES = [(32, 128, 80), (32, 384, 112), (64, 128, 96), (64, 256, 272), (64, 384, 400),
               (64, 512, 80), (64, 640, 64), (64, 768, 96), (64, 896, 32), (64, 1024, 48), (128, 128, 96),
               (64, 64, 48), (64, 192, 208), (64, 320, 64), (64, 448, 96), (64, 576, 80), (64, 704, 32),
               (64, 832, 64), (64, 960, 112),
               (128, 256, 144),
               # chunks with no tiling of their own at that width run as 64-token chunks
               (16, 256, 80), (16, 768, 48), (32, 1024, 64)]


@pytest.mark.parametrize("chunk,dqk,dv", MFMA_SHAPES, ids=lambda v: str(v))
def test_bf16_mfma_tilings(orc, chunk, dqk, dv):
    w = inputs.WORKLOADS["lm_125m"]
    announce(f"fwd bf16 tiling B=1 NH=2 S=256 dqk={dqk} dv={dv} chunk={chunk}")
    from mlstm_matrix_memory_amd import MLSTM_BF16, mlstm_fwd_workspace_bytes
    # a workspace is needed only by the MFMA path: this shape must not fall back to the VALU kernel
    assert mlstm_fwd_workspace_bytes(1, 2, 256, dqk, dv, chunk, MLSTM_BF16) > 0
    x = inputs.fwd_inputs(w, seed=300 + dqk + dv, B=1, NH=2, S=256, dqk=dqk, dv=dv)
    _compare(orc, x, chunk, "bf16")


# the largest widths the boundary accepts (d_qk or d_v = 4096), each against the
# narrowest other width, over three chunks
MAX_WIDTHS = [(4096, 16), (16, 4096)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dqk,dv", MAX_WIDTHS, ids=lambda v: str(v))
def test_maximum_widths(orc, dtype, dqk, dv):
    w = inputs.WORKLOADS["tiny" if dtype == "f32" else "lm_125m"]
    announce(f"fwd {dtype} maximum widths B=1 NH=2 S=96 dqk={dqk} dv={dv} chunk=32")
    x = inputs.fwd_inputs(w, seed=610 + dqk, B=1, NH=2, S=96, dqk=dqk, dv=dv)
    _compare(orc, x, 32, dtype)


# few heads over a long sequence: the scan splits each head's sequence into
# segments chained through their entering states (long-context gate statistics)
SEGMENTED = [(dict(B=1, NH=1, S=2048, dqk=128, dv=96), 64), (dict(B=1, NH=2, S=1024, dqk=384, dv=384), 32),
             (dict(B=1, NH=1, S=4096, dqk=256, dv=256), 128),
             # the streaming form of the scan (widths 512 and 1024), one with a ragged value tile
             (dict(B=1, NH=1, S=2048, dqk=512, dv=512), 64), (dict(B=1, NH=2, S=1024, dqk=1024, dv=112), 64),
             # key widths that are odd multiples of 64 (the segment sums' last key tile half
             # empty), one of them reached by padding 160 to 192
             (dict(B=1, NH=2, S=2048, dqk=64, dv=64), 64), (dict(B=1, NH=1, S=2048, dqk=192, dv=96), 64),
             (dict(B=1, NH=2, S=1024, dqk=320, dv=64), 64), (dict(B=1, NH=1, S=2048, dqk=448, dv=160), 64),
             (dict(B=1, NH=1, S=2048, dqk=160, dv=64), 64)]


@pytest.mark.parametrize("over,chunk", SEGMENTED, ids=lambda v: str(v))
def test_bf16_segmented_sequence(orc, over, chunk):
    w = inputs.WORKLOADS["long_ctx"]
    announce(f"fwd bf16 segmented {over} chunk={chunk}")
    x = inputs.fwd_inputs(w, seed=400 + over["dqk"], **over)
    _compare(orc, x, chunk, "bf16")


# Segments under forget gates close to one (f~ ~ N(8, 1): a chunk keeps about 98%
# of the state), so every token part of a segment reaches the next segment's
# entering state with a weight of order one: the per-part sums of the segment
# states and their decay factors are visible in h and C.  With 256-wide heads the
# first shape runs as 8 segments of 2 token parts each, the second (8 heads, two of
# them compared) as 4 segments of 4 parts.
SEGMENTED_SLOW_DECAY = [(dict(B=1, NH=1, S=4096, dqk=256, dv=256), None),
                        (dict(B=1, NH=8, S=4096, dqk=256, dv=256), (np.array([[0, 0]]), np.array([[1, 6]]))),
                        (dict(B=1, NH=2, S=4096, dqk=64, dv=64), None)]


@pytest.mark.parametrize("over,sel", SEGMENTED_SLOW_DECAY, ids=["1head", "8heads", "2heads_d64"])
def test_bf16_segmented_slow_decay(orc, over, sel):
    w = inputs.WORKLOADS["lm_125m"]
    announce(f"fwd bf16 segmented slow decay {over}")
    x = inputs.fwd_inputs(w, seed=420 + over["NH"], **over)
    x["f_pre"] = x["f_pre"] + np.float32(5.0)
    errs = _compare(orc, x, 64, "bf16", sel=sel)
    print(errs)


FULL = [
    # (batch indices, head indices) of the sampled heads, shaped [1, n] so the
    # selection keeps the [B, NH] leading axes
    ("lm_125m", (np.array([[0, 3, 7]]), np.array([[0, 2, 3]]))),
    ("lm_1_3b", (np.array([[0, 3]]), np.array([[1, 3]]))),
    ("long_ctx", (np.array([[0, 0]]), np.array([[0, 5]]))),
]


@pytest.mark.parametrize("name,sel", FULL, ids=[f[0] for f in FULL])
def test_full_workload_sampled_heads(orc, name, sel):
    w = inputs.WORKLOADS[name]
    announce(f"fwd full workload {name} B={w.B} NH={w.NH} S={w.S} d={w.dqk} chunk={w.chunk}")
    errs = _compare(orc, inputs.fwd_inputs(w), w.chunk, w.dtype, sel=sel)
    print(name, errs)


def test_fwd_is_deterministic():
    w = inputs.WORKLOADS["lm_125m"]
    announce("fwd determinism B=1 NH=2 S=512 d=384")
    x = inputs.fwd_inputs(w, B=1, NH=2, S=512)
    a = fwd_gpu(x, 64, "bf16")
    b = fwd_gpu(x, 64, "bf16")
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_fwd_then_steps_continue_the_sequence(orc):
    """fwd over S tokens, then T mlstm_step calls from its final state == oracle over S+T."""
    import torch
    from gpu_helpers import to_gpu, to_np
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel, mlstm_step
    w = inputs.WORKLOADS["lm_125m"]
    S, T = 256, 6
    announce(f"fwd S={S} then {T} steps, bf16 d=128")
    x = inputs.fwd_inputs(w, seed=77, B=2, NH=2, S=S + T, dqk=128, dv=96)
    dev = {key: to_gpu(val, "bf16" if key in ("q", "k", "v") else "f32") for key, val in x.items()}
    h, C, n, m = mlstm_fwd_parallel(dev["q"][:, :, :S].contiguous(), dev["k"][:, :, :S].contiguous(),
                                    dev["v"][:, :, :S].contiguous(), dev["i_pre"][:, :, :S].contiguous(),
                                    dev["f_pre"][:, :, :S].contiguous(), dev["o_pre"][:, :, :S].contiguous(), 64)
    hs = [to_np(h)]
    for t in range(S, S + T):
        ht = mlstm_step(*(dev[key][:, :, t].contiguous() for key in ("q", "k", "v", "i_pre", "f_pre", "o_pre")),
                        C, n, m)
        hs.append(to_np(ht)[:, :, None, :])
    torch.cuda.synchronize()
    rh, rC, rn, rm = orc.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    errs = {}
    check("h", np.concatenate(hs, axis=2), rh, TOL["bf16"], errs)
    check("C", to_np(C), rC, TOL["bf16"], errs)
    check("n", to_np(n), rn, TOL["bf16"], errs)
    check("m", to_np(m), rm, TOL["bf16"], errs)
