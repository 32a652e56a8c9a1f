"""Helpers for the GPU parity tests: device transfer, the error metric, announcements."""
from __future__ import annotations

import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(msg: str) -> None:
    """Name the case on the real stderr before any GPU work, so a fault still says which."""
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def rel_err(x, r) -> float:
    """max_i |x_i - r_i| / max(|r_i|, RMS(r)) -- relative error floored at the RMS of r."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if r.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    rms = float(np.sqrt(np.mean(r * r)))
    floor = np.maximum(np.abs(r), max(rms, 1e-300))
    return float(np.max(np.abs(x - r) / floor))


def to_gpu(a: np.ndarray, dtype: str):
    """float32 numpy -> torch tensor on cuda:0 (bf16 values are exact by construction)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t


def to_np(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def fwd_gpu(x: dict, chunk: int, dtype: str):
    from mlstm_matrix_memory_amd import mlstm_fwd_parallel
    import torch
    q, k, v = (to_gpu(x[n], dtype) for n in ("q", "k", "v"))
    i_pre, f_pre, o_pre = (to_gpu(x[n], "f32") for n in ("i_pre", "f_pre", "o_pre"))
    h, C, n, m = mlstm_fwd_parallel(q, k, v, i_pre, f_pre, o_pre, chunk)
    torch.cuda.synchronize()
    return to_np(h), to_np(C), to_np(n), to_np(m)


def check(name: str, got, ref, tol: float, errs: dict) -> None:
    e = rel_err(got, ref)
    errs[name] = e
    assert e <= tol, f"{name}: relative error {e:.3e} > {tol:.1e}"


def bwd_gpu(x: dict, dh: np.ndarray, dtype: str):
    """mlstm_bwd_parallel on cuda:0; returns (dq, dk, dv, di, df, do) as float64 numpy."""
    from mlstm_matrix_memory_amd import mlstm_bwd_parallel
    import torch
    q, k, v = (to_gpu(x[n], dtype) for n in ("q", "k", "v"))
    i_pre, f_pre, o_pre = (to_gpu(x[n], "f32") for n in ("i_pre", "f_pre", "o_pre"))
    g = mlstm_bwd_parallel(q, k, v, i_pre, f_pre, o_pre, to_gpu(dh, dtype))
    torch.cuda.synchronize()
    return tuple(to_np(t) for t in g)
