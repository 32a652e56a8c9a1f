"""The kernel's chunkwise decomposition (fp64 numpy model) equals the oracle (CPU only)."""
import numpy as np
import pytest

import oracle
from chunkwise_mirror import chunkwise_forward
from mlstm_matrix_memory_amd import inputs


@pytest.mark.parametrize("chunk", [1, 4, 16, 64, 128, 256])
@pytest.mark.parametrize("name", ["tiny", "long_ctx"])
def test_mirror_matches_oracle_for_every_chunk_size(name, chunk):
    w = inputs.WORKLOADS[name]
    x = inputs.fwd_inputs(w, seed=9, B=1, NH=2, S=256, dqk=16, dv=24)
    h, C, n, m = oracle.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"])
    for hd in range(2):
        args = [x[key][0, hd].astype(np.float64) for key in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
        hm, Cm, nm, mm = chunkwise_forward(*args, chunk)
        np.testing.assert_allclose(hm, h[0, hd], rtol=1e-9, atol=1e-12)
        np.testing.assert_allclose(Cm, C[0, hd], rtol=1e-9, atol=1e-300)
        np.testing.assert_allclose(nm, n[0, hd], rtol=1e-9, atol=1e-300)
        assert abs(mm - m[0, hd]) <= 1e-12 * max(1.0, abs(m[0, hd]))


def test_mirror_with_initial_state_and_ragged_tail():
    w = inputs.WORKLOADS["lm_125m"]
    x = inputs.fwd_inputs(w, seed=3, B=1, NH=1, S=100, dqk=8, dv=8)
    rng = np.random.default_rng(0)
    C0 = rng.standard_normal((1, 1, 8, 8)) * 0.1
    n0 = rng.standard_normal((1, 1, 8))
    m0 = np.array([[2.5]])
    h, C, n, m = oracle.fwd(x["q"], x["k"], x["v"], x["i_pre"], x["f_pre"], x["o_pre"], C0, n0, m0)
    args = [x[key][0, 0].astype(np.float64) for key in ("q", "k", "v", "i_pre", "f_pre", "o_pre")]
    hm, Cm, nm, mm = chunkwise_forward(*args, 32, C0[0, 0], n0[0, 0], m0[0, 0])
    np.testing.assert_allclose(hm, h[0, 0], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(Cm, C[0, 0], rtol=1e-9)
    assert abs(mm - m[0, 0]) < 1e-12
