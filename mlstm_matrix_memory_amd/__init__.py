"""MI355X-native mLSTM matrix-memory cell: HIP kernels behind a C ABI (libmlstm.so).

Entry points (same names as include/mlstm.h):
  mlstm_fwd_parallel  chunkwise parallel forward over whole sequences
  mlstm_fwd_parallel_state
                      the same from a given state, for any sequence length
  mlstm_fwd_parallel_noalloc, mlstm_fwd_noalloc_scratch_bytes
                      mlstm_fwd_parallel for callers that cannot allocate (a per-GPU scratch array)
  mlstm_fwd_prepare, mlstm_fwd_scan
                      the two stages of mlstm_fwd_parallel, for callers that schedule them apart
  mlstm_step          one-token recurrent decode step, state updated in place
  mlstm_bwd_parallel  gradients of the zero-state forward with respect to all inputs
  mlstm_bwd_workspace_bytes
  mlstm_block_epilogue
                      the mLSTM block's per-head GroupNorm, learnable skip and external output gate
  mlstm_fwd_parallel_block, mlstm_fwd_block_workspace_bytes
                      the forward and the block epilogue in one call (fused where a
                      workgroup holds a head's whole rows)
  slstm_fwd           the sLSTM recurrence with block-diagonal (per-head) memory mixing
  mlstm_fwd_workspace_bytes, mlstm_status_string, mlstm_error_detail
"""
from .binding import (  # noqa: F401
    MLSTM_BF16,
    MLSTM_F32,
    MLSTM_FORGET_EXP,
    MLSTM_FORGET_SIGMOID,
    MLSTM_GATE_SIGMOID,
    MLSTM_GATE_SWISH,
    MlstmError,
    load_library,
    mlstm_bwd_parallel,
    mlstm_bwd_workspace_bytes,
    mlstm_block_epilogue,
    mlstm_error_detail,
    mlstm_fwd_block_workspace_bytes,
    mlstm_fwd_noalloc_scratch_bytes,
    mlstm_fwd_parallel,
    mlstm_fwd_parallel_block,
    mlstm_fwd_parallel_noalloc,
    mlstm_fwd_parallel_state,
    mlstm_fwd_prepare,
    mlstm_fwd_scan,
    mlstm_fwd_workspace_bytes,
    mlstm_status_string,
    mlstm_step,
    slstm_fwd,
)
