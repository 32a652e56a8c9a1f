"""The allocation-free forward, mlstm_fwd_parallel_noalloc, against mlstm_fwd_parallel.

Both run the same kernels; the allocation-free one uses the library's per-GPU
scratch array instead of a caller-provided workspace.  Two calls in a row, the
second smaller than the first, must each give exactly what mlstm_fwd_parallel
gives on the same inputs (the scratch keeps the first call's contents, which the
second must not depend on).
"""
import ctypes

import numpy as np
import pytest

from gpu_helpers import announce, to_gpu, to_np
from mlstm_matrix_memory_amd import inputs

pytestmark = pytest.mark.gpu

KEYS = ("q", "k", "v", "i_pre", "f_pre", "o_pre")


def _run_both(over, chunk, seed):
    import torch
    from mlstm_matrix_memory_amd import MLSTM_BF16, binding, mlstm_fwd_parallel
    w = inputs.WORKLOADS["lm_125m"]
    x = inputs.fwd_inputs(w, seed=seed, **over)
    dev = [to_gpu(x[key], "bf16" if key in ("q", "k", "v") else "f32") for key in KEYS]
    B, NH, S, dqk = dev[0].shape
    dv = dev[2].shape[-1]
    ref = mlstm_fwd_parallel(*dev, chunk)
    torch.cuda.synchronize()
    out = [torch.full_like(t, float("nan")) for t in ref]
    lib = binding.load_library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.mlstm_fwd_parallel_noalloc(*(t.data_ptr() for t in dev), B, NH, S, dqk, dv, chunk, MLSTM_BF16,
                                        *(t.data_ptr() for t in out), stream)
    assert st == 0, binding.mlstm_error_detail()
    torch.cuda.synchronize()
    for name, a, b in zip(("h", "C", "n", "m"), ref, out):
        ra, rb = to_np(a), to_np(b)
        assert np.all(np.isfinite(rb)), f"{name} is not finite"
        assert np.array_equal(ra, rb), f"{name}: max difference {np.max(np.abs(ra - rb))}"


def test_noalloc_two_calls_second_smaller():
    announce("fwd noalloc: B=2 NH=4 S=1024 d=384 chunk=64, then B=1 NH=2 S=256 d=128 chunk=32")
    _run_both(dict(B=2, NH=4, S=1024), 64, 820)
    _run_both(dict(B=1, NH=2, S=256, dqk=128, dv=96), 32, 821)


def test_noalloc_streaming_scan_two_calls_second_smaller():
    # widths 1024 and 512 run the streaming form of the scan, whose workspace also
    # holds the operand-ordered copies of q and k
    announce("fwd noalloc: B=1 NH=4 S=512 d=1024 chunk=64, then B=1 NH=2 S=256 d=512 chunk=64")
    _run_both(dict(B=1, NH=4, S=512, dqk=1024, dv=1024), 64, 822)
    _run_both(dict(B=1, NH=2, S=256, dqk=512, dv=512), 64, 823)


def test_noalloc_padded_key_width_two_calls_second_smaller():
    # a key width that is not a multiple of 64 runs on zero-padded copies of q and k,
    # which the scratch also holds
    announce("fwd noalloc: B=1 NH=2 S=512 dqk=96 dv=80 chunk=64, then B=1 NH=1 S=256 dqk=48 dv=64 chunk=64")
    _run_both(dict(B=1, NH=2, S=512, dqk=96, dv=80), 64, 824)
    _run_both(dict(B=1, NH=1, S=256, dqk=48, dv=64), 64, 825)


def test_noalloc_rejects_a_forward_larger_than_its_scratch():
    from mlstm_matrix_memory_amd import MLSTM_BF16, binding
    lib = binding.load_library()
    cap = binding.mlstm_fwd_noalloc_scratch_bytes()
    assert binding.mlstm_fwd_workspace_bytes(8, 32, 2048, 384, 384, 64, MLSTM_BF16) > cap
    st = lib.mlstm_fwd_parallel_noalloc(*([0x10000] * 6), 8, 32, 2048, 384, 384, 64, MLSTM_BF16,
                                        *([0x10000] * 4), None)
    assert st == binding.MLSTM_ERR_UNSUPPORTED
    assert "scratch" in binding.mlstm_error_detail()
