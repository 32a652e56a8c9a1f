"""Input generator recipe checks and the oracle regression fixture (CPU only)."""
import json
import math
import os

import numpy as np
import torch

import oracle
from mlstm_matrix_memory_amd import inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_round_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.3895314e38], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = inputs.bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # bits round trip
    bits = inputs.bf16_bits(got)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back.view(np.uint32), got.view(np.uint32))


def test_workload_shapes_and_determinism():
    w = inputs.WORKLOADS["tiny"]
    a = inputs.fwd_inputs(w)
    b = inputs.fwd_inputs(w)
    for key in a:
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (1, 1, 64, 16) and a["o_pre"].shape == (1, 1, 64, 16)
    assert a["i_pre"].shape == (1, 1, 64)
    # k scaled by 1/sqrt(d_qk)
    assert abs(float(np.std(a["k"])) * math.sqrt(16) - 1.0) < 0.3


def test_long_ctx_spikes_and_bf16():
    w = inputs.WORKLOADS["long_ctx"]
    x = inputs.fwd_inputs(w, S=4096, NH=2, dqk=32, dv=32)
    n_spikes = int(np.sum(x["i_pre"] == np.float32(40.0)))
    assert n_spikes == math.floor(0.01 * 2 * 4096)
    assert np.array_equal(inputs.bf16_round(x["q"]), x["q"])


def test_decode_state_distribution():
    w = inputs.WORKLOADS["decode"]
    st = inputs.step_state(w, B=4, NH=2, dqk=64, dv=32)
    assert st["C"].shape == (4, 2, 32, 64)
    assert 0.0 <= st["m"].min() and st["m"].max() < 5.0
    assert abs(float(np.std(st["C"])) * 64 - 1.0) < 0.1


def test_oracle_regression_fixture():
    ref = json.load(open(os.path.join(HERE, "golden", "tiny_oracle.json")))
    x = inputs.fwd_inputs(inputs.WORKLOADS["tiny"])
    h, C, n, m = oracle.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    for ix, val in ref["h_samples"]:
        assert math.isclose(h[tuple(ix)], val, rel_tol=1e-12, abs_tol=1e-15)
    assert math.isclose(float(h.sum()), ref["h_sum"], rel_tol=1e-11)
    assert math.isclose(float(C.sum()), ref["C_sum"], rel_tol=1e-11)
    assert math.isclose(float(n.sum()), ref["n_sum"], rel_tol=1e-11)
    assert math.isclose(float(m[0, 0]), ref["m"], rel_tol=1e-13)
