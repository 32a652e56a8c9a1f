"""ctypes binding of libmlstm (include/mlstm.h), same names as the C entry points.

Argument marshalling only: this module checks tensor dtypes, shapes, devices and
contiguity, allocates outputs and workspace with torch (device memory and the
current stream are the only things torch provides), and passes raw pointers to
the C ABI.  Every step of the mLSTM cell runs in the HIP kernels of
``libmlstm.so``; there is no other implementation behind these functions, and
they raise if the library is not built.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libmlstm.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "mlstm.h")

MLSTM_OK = 0
MLSTM_ERR_INVALID_ARG = 1
MLSTM_ERR_UNSUPPORTED = 2
MLSTM_ERR_WORKSPACE = 3
MLSTM_ERR_HIP = 4

MLSTM_F32 = 0
MLSTM_BF16 = 1

_lib = None


class MlstmError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        self.status = status
        self.detail = detail
        super().__init__(f"{fn}: {mlstm_status_string(status)} ({status}): {detail}")


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libmlstm.so; raises if it has not been built (no fallback exists).

    torch is imported first.  The library's HIP runtime dependency
    (libamdhip64.so.7) then binds to the runtime torch has already loaded, so the
    device pointers and streams torch hands over belong to the runtime that
    launches the kernels.  Loaded before torch, the library would bring up a
    second HIP runtime beside torch's, which does not see the device."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                           "or `python mlstm_matrix_memory_amd/build.py`")
    import torch  # noqa: F401  (loads torch's HIP runtime before the library's dependency is resolved)
    lib = ctypes.CDLL(path)
    vp, fp, i, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mlstm_fwd_workspace_bytes.restype = sz
    lib.mlstm_fwd_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.mlstm_fwd_parallel.restype = i
    lib.mlstm_fwd_parallel.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i,
                                       vp, fp, fp, fp, vp, sz, vp]
    lib.mlstm_fwd_parallel_state.restype = i
    lib.mlstm_fwd_parallel_state.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i,
                                             fp, fp, fp, vp, fp, fp, fp, vp, sz, vp]
    lib.mlstm_fwd_noalloc_scratch_bytes.restype = sz
    lib.mlstm_fwd_noalloc_scratch_bytes.argtypes = []
    lib.mlstm_fwd_parallel_noalloc.restype = i
    lib.mlstm_fwd_parallel_noalloc.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i,
                                               vp, fp, fp, fp, vp]
    lib.mlstm_fwd_prepare.restype = i
    lib.mlstm_fwd_prepare.argtypes = [vp, vp, fp, fp, i, i, i, i, i, i, i, vp, sz, vp]
    lib.mlstm_fwd_scan.restype = i
    lib.mlstm_fwd_scan.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, i, i,
                                   vp, fp, fp, fp, vp, sz, vp]
    lib.mlstm_bwd_workspace_bytes.restype = sz
    lib.mlstm_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.mlstm_bwd_parallel.restype = i
    lib.mlstm_bwd_parallel.argtypes = [vp, vp, vp, fp, fp, fp, vp, i, i, i, i, i, i,
                                       fp, fp, fp, fp, fp, fp, vp, sz, vp]
    lib.mlstm_fwd_block_workspace_bytes.restype = sz
    lib.mlstm_fwd_block_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i]
    lib.mlstm_fwd_parallel_block.restype = i
    lib.mlstm_fwd_parallel_block.argtypes = [vp, vp, vp, fp, fp, fp, vp, vp, fp, fp, fp, i, i, i, i, i, i,
                                             ctypes.c_float, i, i, i, vp, fp, fp, fp, vp, sz, vp]
    lib.mlstm_block_epilogue.restype = i
    lib.mlstm_block_epilogue.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, ctypes.c_float, i, i, vp, vp]
    lib.slstm_fwd.restype = i
    lib.slstm_fwd.argtypes = [fp, vp, i, i, i, i, i, i, fp, fp, fp, fp, vp, fp, fp, fp, fp, vp]
    lib.mlstm_step.restype = i
    lib.mlstm_step.argtypes = [vp, vp, vp, fp, fp, fp, i, i, i, i, i, fp, fp, fp, vp, vp]
    lib.mlstm_status_string.restype = ctypes.c_char_p
    lib.mlstm_status_string.argtypes = [i]
    lib.mlstm_error_detail.restype = ctypes.c_char_p
    lib.mlstm_error_detail.argtypes = []
    if path == LIBRARY:
        _lib = lib
    return lib


def header_symbols(path: str = HEADER) -> list[str]:
    """Names of the functions include/mlstm.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mlstm|slstm)_[a-z_0-9]+)\s*\(", text)))


def mlstm_status_string(status: int) -> str:
    return load_library().mlstm_status_string(int(status)).decode()


def mlstm_error_detail() -> str:
    return load_library().mlstm_error_detail().decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return MLSTM_F32
    if t.dtype == torch.bfloat16:
        return MLSTM_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def mlstm_fwd_workspace_bytes(B: int, NH: int, S: int, d_qk: int, d_v: int, chunk: int, dtype: int) -> int:
    return int(load_library().mlstm_fwd_workspace_bytes(B, NH, S, d_qk, d_v, chunk, int(dtype)))


def _check(t, name, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _keep_for_stream(stream, device, tensors):
    """Tensors a wrapper allocated itself (workspace, outputs) are allocated on the
    current stream but used by kernels enqueued on `stream`.  When that is another
    stream, tell torch's caching allocator, so that it does not hand their memory to
    a later allocation on the current stream while those kernels still run."""
    import torch
    if stream is None or stream == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _fwd_args(q, k, v, i_pre, f_pre, o_pre, chunk, h_out, C_final, n_final, m_final, workspace, need_outputs,
              stream=None):
    """Checks the forward's tensors, allocates what is missing; returns the argument tuple."""
    import torch
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, NH, S, d]")
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(q)
    _check(q, "q", (B, NH, S, dqk), q.dtype, dev)
    _check(k, "k", (B, NH, S, dqk), q.dtype, dev)
    _check(v, "v", (B, NH, S, dv), q.dtype, dev)
    _check(i_pre, "i_pre", (B, NH, S), torch.float32, dev)
    _check(f_pre, "f_pre", (B, NH, S), torch.float32, dev)
    _check(o_pre, "o_pre", (B, NH, S, dv), torch.float32, dev)
    owned = []            # tensors allocated here, used by kernels on `stream`
    if need_outputs:
        if h_out is None:
            h_out = torch.empty((B, NH, S, dv), dtype=q.dtype, device=dev)
            owned.append(h_out)
        if C_final is None:
            C_final = torch.empty((B, NH, dv, dqk), dtype=torch.float32, device=dev)
            owned.append(C_final)
        if n_final is None:
            n_final = torch.empty((B, NH, dqk), dtype=torch.float32, device=dev)
            owned.append(n_final)
        if m_final is None:
            m_final = torch.empty((B, NH), dtype=torch.float32, device=dev)
            owned.append(m_final)
        _check(h_out, "h_out", (B, NH, S, dv), q.dtype, dev)
        _check(C_final, "C_final", (B, NH, dv, dqk), torch.float32, dev)
        _check(n_final, "n_final", (B, NH, dqk), torch.float32, dev)
        _check(m_final, "m_final", (B, NH), torch.float32, dev)
    need = int(lib.mlstm_fwd_workspace_bytes(B, NH, S, dqk, dv, chunk, dt))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        owned.append(workspace)
    _keep_for_stream(stream, dev, owned)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return (B, NH, S, dqk, dv, dt, h_out, C_final, n_final, m_final, workspace, ws_ptr, ws_bytes, dev)


def mlstm_fwd_parallel(q, k, v, i_pre, f_pre, o_pre, chunk: int,
                       h_out=None, C_final=None, n_final=None, m_final=None,
                       workspace=None, stream=None):
    """Chunkwise parallel forward from the zero state; returns (h, C, n, m).

    q,k [B,NH,S,d_qk] and v [B,NH,S,d_v] float32 or bfloat16 on one GPU;
    i_pre,f_pre [B,NH,S] and o_pre [B,NH,S,d_v] float32.  Outputs are allocated
    when not given: h like v, C [B,NH,d_v,d_qk], n [B,NH,d_qk], m [B,NH] float32.
    """
    lib = load_library()
    (B, NH, S, dqk, dv, dt, h_out, C_final, n_final, m_final, workspace, ws_ptr, ws_bytes, dev) = _fwd_args(
        q, k, v, i_pre, f_pre, o_pre, chunk, h_out, C_final, n_final, m_final, workspace, True, stream)
    st = lib.mlstm_fwd_parallel(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                                B, NH, S, dqk, dv, int(chunk), dt,
                                h_out.data_ptr(), C_final.data_ptr(), n_final.data_ptr(), m_final.data_ptr(),
                                ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_parallel", st, mlstm_error_detail())
    return h_out, C_final, n_final, m_final


def mlstm_fwd_block_workspace_bytes(B: int, NH: int, S: int, d_qk: int, d_v: int, chunk: int, dtype: int,
                                    fuse: int = 0) -> int:
    return int(load_library().mlstm_fwd_block_workspace_bytes(B, NH, S, d_qk, d_v, chunk, dtype, int(fuse)))


def mlstm_fwd_parallel_block(q, k, v, i_pre, f_pre, o_pre, x, z, gn_weight, gn_bias, skip_weight, chunk: int,
                             eps: float = 1e-5, act: int = 0, fuse: int = 0, y_out=None, C_final=None,
                             n_final=None, m_final=None, workspace=None, stream=None):
    """Zero-state forward followed by the block epilogue; returns (y, C, n, m).

    The inputs of mlstm_fwd_parallel, plus x, z like v and gn_weight, gn_bias,
    skip_weight [NH,d_v] float32 (see mlstm_block_epilogue); h is not returned.
    fuse=1 applies the epilogue inside the scan where the tiling allows it.
    """
    import torch
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, NH, S, d]")
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(q)
    for t, name, shape, dtype in ((q, "q", (B, NH, S, dqk), q.dtype), (k, "k", (B, NH, S, dqk), q.dtype),
                                  (v, "v", (B, NH, S, dv), q.dtype), (i_pre, "i_pre", (B, NH, S), torch.float32),
                                  (f_pre, "f_pre", (B, NH, S), torch.float32),
                                  (o_pre, "o_pre", (B, NH, S, dv), torch.float32),
                                  (x, "x", (B, NH, S, dv), q.dtype), (z, "z", (B, NH, S, dv), q.dtype),
                                  (gn_weight, "gn_weight", (NH, dv), torch.float32),
                                  (gn_bias, "gn_bias", (NH, dv), torch.float32),
                                  (skip_weight, "skip_weight", (NH, dv), torch.float32)):
        _check(t, name, shape, dtype, dev)
    owned = []
    if y_out is None:
        y_out = torch.empty((B, NH, S, dv), dtype=q.dtype, device=dev)
        owned.append(y_out)
    if C_final is None:
        C_final = torch.empty((B, NH, dv, dqk), dtype=torch.float32, device=dev)
        owned.append(C_final)
    if n_final is None:
        n_final = torch.empty((B, NH, dqk), dtype=torch.float32, device=dev)
        owned.append(n_final)
    if m_final is None:
        m_final = torch.empty((B, NH), dtype=torch.float32, device=dev)
        owned.append(m_final)
    _check(y_out, "y_out", (B, NH, S, dv), q.dtype, dev)
    _check(C_final, "C_final", (B, NH, dv, dqk), torch.float32, dev)
    _check(n_final, "n_final", (B, NH, dqk), torch.float32, dev)
    _check(m_final, "m_final", (B, NH), torch.float32, dev)
    need = int(lib.mlstm_fwd_block_workspace_bytes(B, NH, S, dqk, dv, int(chunk), dt, int(fuse)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        owned.append(workspace)
    _keep_for_stream(stream, dev, owned)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.mlstm_fwd_parallel_block(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                                      x.data_ptr(), z.data_ptr(), gn_weight.data_ptr(), gn_bias.data_ptr(),
                                      skip_weight.data_ptr(), B, NH, S, dqk, dv, int(chunk), float(eps), int(act),
                                      dt, int(fuse), y_out.data_ptr(), C_final.data_ptr(), n_final.data_ptr(),
                                      m_final.data_ptr(), ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_parallel_block", st, mlstm_error_detail())
    return y_out, C_final, n_final, m_final


def mlstm_fwd_noalloc_scratch_bytes() -> int:
    return int(load_library().mlstm_fwd_noalloc_scratch_bytes())


def mlstm_fwd_parallel_noalloc(q, k, v, i_pre, f_pre, o_pre, chunk: int, h_out, C_final, n_final, m_final,
                               stream=None):
    """mlstm_fwd_parallel without a workspace: the library's per-GPU scratch array
    serves instead, and nothing is allocated here either (outputs are required).
    Calls that overlap in time on one GPU race on that array."""
    import torch
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, NH, S, d]")
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(q)
    for t, name, shp, tdt in ((q, "q", (B, NH, S, dqk), q.dtype), (k, "k", (B, NH, S, dqk), q.dtype),
                              (v, "v", (B, NH, S, dv), q.dtype), (i_pre, "i_pre", (B, NH, S), torch.float32),
                              (f_pre, "f_pre", (B, NH, S), torch.float32),
                              (o_pre, "o_pre", (B, NH, S, dv), torch.float32),
                              (h_out, "h_out", (B, NH, S, dv), q.dtype),
                              (C_final, "C_final", (B, NH, dv, dqk), torch.float32),
                              (n_final, "n_final", (B, NH, dqk), torch.float32),
                              (m_final, "m_final", (B, NH), torch.float32)):
        if t is None:
            raise ValueError(f"{name} is required (this entry point allocates nothing)")
        _check(t, name, shp, tdt, dev)
    st = lib.mlstm_fwd_parallel_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                        i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                                        B, NH, S, dqk, dv, int(chunk), dt,
                                        h_out.data_ptr(), C_final.data_ptr(), n_final.data_ptr(),
                                        m_final.data_ptr(), _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_parallel_noalloc", st, mlstm_error_detail())
    return h_out, C_final, n_final, m_final


def mlstm_fwd_parallel_state(q, k, v, i_pre, f_pre, o_pre, chunk: int, C_init=None, n_init=None, m_init=None,
                             h_out=None, C_final=None, n_final=None, m_final=None,
                             workspace=None, stream=None):
    """Chunkwise parallel forward from a given stabilized state, any S >= 1; returns (h, C, n, m).

    Like mlstm_fwd_parallel; C_init [B,NH,d_v,d_qk], n_init [B,NH,d_qk], m_init [B,NH]
    float32 give the state entering the first token (all None = zero state) and
    must not share memory with the final state.
    """
    import torch
    lib = load_library()
    (B, NH, S, dqk, dv, dt, h_out, C_final, n_final, m_final, workspace, ws_ptr, ws_bytes, dev) = _fwd_args(
        q, k, v, i_pre, f_pre, o_pre, chunk, h_out, C_final, n_final, m_final, workspace, True, stream)
    given = [t is not None for t in (C_init, n_init, m_init)]
    if any(given):
        if not all(given):
            raise ValueError("C_init, n_init and m_init must be given together")
        _check(C_init, "C_init", (B, NH, dv, dqk), torch.float32, dev)
        _check(n_init, "n_init", (B, NH, dqk), torch.float32, dev)
        _check(m_init, "m_init", (B, NH), torch.float32, dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = lib.mlstm_fwd_parallel_state(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                      i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                                      B, NH, S, dqk, dv, int(chunk), dt,
                                      ptr(C_init), ptr(n_init), ptr(m_init),
                                      h_out.data_ptr(), C_final.data_ptr(), n_final.data_ptr(), m_final.data_ptr(),
                                      ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_parallel_state", st, mlstm_error_detail())
    return h_out, C_final, n_final, m_final


def mlstm_fwd_prepare(q, k, v, i_pre, f_pre, o_pre, chunk: int, workspace, stream=None):
    """First stage of mlstm_fwd_parallel (per-chunk gates and decayed scores into workspace)."""
    lib = load_library()
    (B, NH, S, dqk, dv, dt, _, _, _, _, workspace, ws_ptr, ws_bytes, dev) = _fwd_args(
        q, k, v, i_pre, f_pre, o_pre, chunk, None, None, None, None, workspace, False, stream)
    st = lib.mlstm_fwd_prepare(q.data_ptr(), k.data_ptr(), i_pre.data_ptr(), f_pre.data_ptr(),
                               B, NH, S, dqk, dv, int(chunk), dt, ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_prepare", st, mlstm_error_detail())


def mlstm_fwd_scan(q, k, v, i_pre, f_pre, o_pre, chunk: int, h_out, C_final, n_final, m_final,
                   workspace, stream=None):
    """Second stage of mlstm_fwd_parallel (sequential pass over chunks); outputs given."""
    lib = load_library()
    (B, NH, S, dqk, dv, dt, h_out, C_final, n_final, m_final, workspace, ws_ptr, ws_bytes, dev) = _fwd_args(
        q, k, v, i_pre, f_pre, o_pre, chunk, h_out, C_final, n_final, m_final, workspace, True, stream)
    st = lib.mlstm_fwd_scan(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                            i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                            B, NH, S, dqk, dv, int(chunk), dt,
                            h_out.data_ptr(), C_final.data_ptr(), n_final.data_ptr(), m_final.data_ptr(),
                            ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_fwd_scan", st, mlstm_error_detail())
    return h_out, C_final, n_final, m_final


def mlstm_bwd_workspace_bytes(B: int, NH: int, S: int, d_qk: int, d_v: int, dtype: int) -> int:
    return int(load_library().mlstm_bwd_workspace_bytes(B, NH, S, d_qk, d_v, int(dtype)))


def mlstm_bwd_parallel(q, k, v, i_pre, f_pre, o_pre, dh, grads=None, workspace=None, stream=None):
    """Gradients of the zero-state forward given dh; returns (dq, dk, dv, di, df, do), float32.

    Inputs as for mlstm_fwd_parallel; dh [B,NH,S,d_v] in the dtype of q.  `grads`
    may hold the six output tensors (float32, shapes of q, k, v, i_pre, f_pre, o_pre).
    """
    import torch
    lib = load_library()
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, NH, S, d]")
    B, NH, S, dqk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(q)
    shapes = [(B, NH, S, dqk), (B, NH, S, dqk), (B, NH, S, dv), (B, NH, S), (B, NH, S), (B, NH, S, dv)]
    for t, name, shp, tdt in zip((q, k, v, i_pre, f_pre, o_pre, dh), ("q", "k", "v", "i_pre", "f_pre", "o_pre", "dh"),
                                 shapes + [(B, NH, S, dv)], [q.dtype] * 3 + [torch.float32] * 3 + [q.dtype]):
        _check(t, name, shp, tdt, dev)
    owned = []
    if grads is None:
        grads = tuple(torch.empty(shp, dtype=torch.float32, device=dev) for shp in shapes)
        owned.extend(grads)
    for t, name, shp in zip(grads, ("grad_q", "grad_k", "grad_v", "grad_i", "grad_f", "grad_o"), shapes):
        _check(t, name, shp, torch.float32, dev)
    need = int(lib.mlstm_bwd_workspace_bytes(B, NH, S, dqk, dv, dt))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        owned.append(workspace)
    _keep_for_stream(stream, dev, owned)
    st = lib.mlstm_bwd_parallel(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(), dh.data_ptr(),
                                B, NH, S, dqk, dv, dt, *[g.data_ptr() for g in grads],
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_bwd_parallel", st, mlstm_error_detail())
    return tuple(grads)


MLSTM_GATE_SIGMOID = 0
MLSTM_GATE_SWISH = 1


def mlstm_block_epilogue(h, x, z, gn_weight, gn_bias, skip_weight, eps: float = 1e-5,
                         act: int = MLSTM_GATE_SIGMOID, y_out=None, stream=None):
    """Per-head GroupNorm of h, plus skip_weight * x, gated by act(z); returns y.

    h, x, z [B,NH,S,d_v] float32 or bfloat16 (one dtype); gn_weight, gn_bias,
    skip_weight [NH,d_v] float32; y_out like h (may be h, x or z itself).
    """
    import torch
    lib = load_library()
    if h.dim() != 4:
        raise ValueError("h must be 4-D [B, NH, S, d_v]")
    B, NH, S, dv = h.shape
    dev = h.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(h)
    for t, name in ((h, "h"), (x, "x"), (z, "z")):
        _check(t, name, (B, NH, S, dv), h.dtype, dev)
    for t, name in ((gn_weight, "gn_weight"), (gn_bias, "gn_bias"), (skip_weight, "skip_weight")):
        _check(t, name, (NH, dv), torch.float32, dev)
    if y_out is None:
        y_out = torch.empty_like(h)
        _keep_for_stream(stream, dev, [y_out])
    _check(y_out, "y_out", (B, NH, S, dv), h.dtype, dev)
    st = lib.mlstm_block_epilogue(h.data_ptr(), x.data_ptr(), z.data_ptr(), gn_weight.data_ptr(),
                                  gn_bias.data_ptr(), skip_weight.data_ptr(), B, NH, S, dv, float(eps), int(act),
                                  dt, y_out.data_ptr(), _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_block_epilogue", st, mlstm_error_detail())
    return y_out


MLSTM_FORGET_SIGMOID = 0
MLSTM_FORGET_EXP = 1


def slstm_fwd(x_pre, R, forget: int = MLSTM_FORGET_SIGMOID, c_init=None, n_init=None, m_init=None, h_init=None,
              h_out=None, c_final=None, n_final=None, m_final=None, h_final=None, stream=None):
    """sLSTM recurrence; returns (h [B,NH,S,d_h], c, n, m, h_last [B,NH,d_h]).

    x_pre [B,NH,S,4,d_h] float32 (gates z, i, f, o); R [NH,4,d_h,d_h] float32 or
    bfloat16 (also the dtype of h); states [B,NH,d_h] float32, all four or none.
    """
    import torch
    lib = load_library()
    if x_pre.dim() != 5 or x_pre.shape[3] != 4:
        raise ValueError("x_pre must be [B, NH, S, 4, d_h]")
    B, NH, S, _, dh = x_pre.shape
    dev = x_pre.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(R)
    _check(x_pre, "x_pre", (B, NH, S, 4, dh), torch.float32, dev)
    _check(R, "R", (NH, 4, dh, dh), R.dtype, dev)
    init = [c_init, n_init, m_init, h_init]
    if any(t is not None for t in init):
        if not all(t is not None for t in init):
            raise ValueError("c_init, n_init, m_init and h_init must be given together")
        for t, name in zip(init, ("c_init", "n_init", "m_init", "h_init")):
            _check(t, name, (B, NH, dh), torch.float32, dev)
    owned = []
    if h_out is None:
        h_out = torch.empty((B, NH, S, dh), dtype=R.dtype, device=dev)
        owned.append(h_out)
    fin = [c_final, n_final, m_final, h_final]
    for j, t in enumerate(fin):
        if t is None:
            fin[j] = torch.empty((B, NH, dh), dtype=torch.float32, device=dev)
            owned.append(fin[j])
    _keep_for_stream(stream, dev, owned)
    _check(h_out, "h_out", (B, NH, S, dh), R.dtype, dev)
    for t, name in zip(fin, ("c_final", "n_final", "m_final", "h_final")):
        _check(t, name, (B, NH, dh), torch.float32, dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    st = lib.slstm_fwd(x_pre.data_ptr(), R.data_ptr(), B, NH, S, dh, int(forget), dt, *[ptr(t) for t in init],
                       h_out.data_ptr(), *[t.data_ptr() for t in fin], _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("slstm_fwd", st, mlstm_error_detail())
    return (h_out, *fin)


def mlstm_step(q, k, v, i_pre, f_pre, o_pre, C, n, m, h_out=None, stream=None):
    """One recurrent step; (C, n, m) are updated in place.  Returns h [B,NH,d_v].

    q,k [B,NH,d_qk], v [B,NH,d_v] float32 or bfloat16; i_pre,f_pre [B,NH] and
    o_pre [B,NH,d_v] float32; C [B,NH,d_v,d_qk], n [B,NH,d_qk], m [B,NH] float32.
    """
    import torch
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be 3-D [B, NH, d]")
    B, NH, dqk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a GPU")
    dt = _dtype_code(q)
    _check(q, "q", (B, NH, dqk), q.dtype, dev)
    _check(k, "k", (B, NH, dqk), q.dtype, dev)
    _check(v, "v", (B, NH, dv), q.dtype, dev)
    _check(i_pre, "i_pre", (B, NH), torch.float32, dev)
    _check(f_pre, "f_pre", (B, NH), torch.float32, dev)
    _check(o_pre, "o_pre", (B, NH, dv), torch.float32, dev)
    _check(C, "C", (B, NH, dv, dqk), torch.float32, dev)
    _check(n, "n", (B, NH, dqk), torch.float32, dev)
    _check(m, "m", (B, NH), torch.float32, dev)
    if h_out is None:
        h_out = torch.empty((B, NH, dv), dtype=q.dtype, device=dev)
        _keep_for_stream(stream, dev, [h_out])
    _check(h_out, "h_out", (B, NH, dv), q.dtype, dev)
    st = lib.mlstm_step(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                        i_pre.data_ptr(), f_pre.data_ptr(), o_pre.data_ptr(),
                        B, NH, dqk, dv, dt,
                        C.data_ptr(), n.data_ptr(), m.data_ptr(), h_out.data_ptr(),
                        _stream_handle(stream, dev))
    if st != MLSTM_OK:
        raise MlstmError("mlstm_step", st, mlstm_error_detail())
    return h_out
