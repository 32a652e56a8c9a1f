"""GPU parity of slstm_fwd against the fp64 oracle's sLSTM recurrence.

Small cases compare every output; the slstm_125m workload (B=8, NH=4, S=2048,
d_h=192) runs whole and the oracle recomputes all of it (O(S d_h^2) per sequence).
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


def _run(x, dtype, forget, state=None):
    import torch
    from mlstm_matrix_memory_amd import slstm_fwd
    xp = to_gpu(x["x_pre"], "f32")
    R = to_gpu(x["R"], dtype)
    st = [to_gpu(a, "f32") for a in state] if state is not None else [None] * 4
    out = slstm_fwd(xp, R, forget, *st)
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in out)


def _compare(orc, x, dtype, forget=0, state=None):
    got = _run(x, dtype, forget, state)
    ref = orc.slstm(x["x_pre"], x["R"], forget, *(state if state is not None else []))
    ref = list(ref)
    errs = {}
    if dtype == "bf16":
        # h against the oracle itself here, and below against its output rounded as h is stored
        check("h_unrounded", got[0], ref[0], TOL[dtype], errs)
        ref[0] = inputs.bf16_round(ref[0].astype(np.float32)).astype(np.float64)
    # c and n are the stabilized states (c e^{-m}, n e^{-m}); once m matches, each is
    # fixed on its own, so each is compared, and so is their ratio (what h is made of)
    check("h", got[0], ref[0], TOL[dtype], errs)
    check("c", got[1], ref[1], TOL[dtype], errs)
    check("n", got[2], ref[2], TOL[dtype], errs)
    check("c/n", got[1] / got[2], ref[1] / ref[2], TOL[dtype], errs)
    check("m", got[3], ref[3], TOL[dtype], errs)
    check("h_last", got[4], ref[4], TOL[dtype], errs)
    return got


@pytest.mark.parametrize("forget", [0, 1])
@pytest.mark.parametrize("dh", [16, 48, 64, 128])
def test_fp32(orc, dh, forget):
    w = inputs.WORKLOADS["slstm_125m"]
    announce(f"slstm fp32 B=3 NH=2 S=70 dh={dh} forget={forget}")
    x = inputs.slstm_inputs(w, seed=600 + dh, B=3, NH=2, S=70, dh=dh)
    _compare(orc, x, "f32", forget)


@pytest.mark.parametrize("dh", [32, 96, 160, 192])
def test_bf16_widths(orc, dh):
    w = inputs.WORKLOADS["slstm_125m"]
    announce(f"slstm bf16 B=9 NH=2 S=120 dh={dh}")
    # B=9: two full tiles of 4 sequences and a tile with one
    x = inputs.slstm_inputs(w, seed=620 + dh, B=9, NH=2, S=120, dh=dh)
    _compare(orc, x, "bf16", 0)


def test_bf16_full_size(orc):
    w = inputs.WORKLOADS["slstm_125m"]
    announce("slstm bf16 slstm_125m full size")
    _compare(orc, inputs.slstm_inputs(w), "bf16", 0)


def test_continuation(orc):
    # two calls, the second from the state the first returned, equal one call
    w = inputs.WORKLOADS["slstm_125m"]
    announce("slstm fp32 continuation B=2 NH=2 S=50 dh=64")
    x = inputs.slstm_inputs(w, seed=640, B=2, NH=2, S=50, dh=64)
    first = _run({"x_pre": x["x_pre"][:, :, :20], "R": x["R"]}, "f32", 0)
    second = {"x_pre": x["x_pre"][:, :, 20:], "R": x["R"]}
    got = _compare(orc, second, "f32", 0, state=first[1:])
    ref = orc.slstm(x["x_pre"], x["R"], 0)
    errs = {}
    check("h continued", got[0], ref[0][:, :, 20:], TOL["f32"], errs)


def test_in_place_state():
    import torch
    from mlstm_matrix_memory_amd import slstm_fwd
    w = inputs.WORKLOADS["slstm_125m"]
    announce("slstm bf16 in-place state B=2 NH=1 S=30 dh=64")
    x = inputs.slstm_inputs(w, seed=650, B=2, NH=1, S=30, dh=64)
    xp, R = to_gpu(x["x_pre"], "f32"), to_gpu(x["R"], "bf16")
    h1, c, n, m, hl = slstm_fwd(xp[:, :, :10].contiguous(), R)
    c2, n2, m2, hl2 = c.clone(), n.clone(), m.clone(), hl.clone()
    ref = slstm_fwd(xp[:, :, 10:].contiguous(), R, 0, c, n, m, hl)
    slstm_fwd(xp[:, :, 10:].contiguous(), R, 0, c2, n2, m2, hl2, c_final=c2, n_final=n2, m_final=m2, h_final=hl2)
    torch.cuda.synchronize()
    for a, b in zip(ref[1:], (c2, n2, m2, hl2)):
        assert torch.equal(a, b)
