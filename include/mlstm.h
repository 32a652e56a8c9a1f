/*
 * mlstm.h -- C ABI of libmlstm: the mLSTM matrix-memory cell on AMD Instinct
 * MI355X (gfx950).
 *
 * Method: "xLSTM: Extended Long Short-Term Memory" (arXiv 2405.04517).
 *   - section 2.3 "mLSTM", eq. (18): the memory of each head is a matrix C that
 *     stores a key/value pair by the covariance update C_t = C_{t-1} + v_t k_t^T;
 *     the forget gate is the decay rate applied to C_{t-1}, the input gate the
 *     learning rate applied to v_t k_t^T, the output gate scales the retrieved
 *     vector;
 *   - section 2.3, normalizer paragraph: n_t is the input-gate and forget-gate
 *     weighted sum of keys; retrieval divides C_t q_t by max(|n_t^T q_t|, 1.0);
 *   - section 2.2, stabilizer paragraph and eq. (17): a log-domain state m_t keeps
 *     the exponential input gate from overflowing, and using the stabilized gates
 *     f'_t, i'_t changes no output;
 *   - section 2.3, multi-head paragraph: heads do not mix, and the recurrence has an
 *     equivalent parallel (chunkwise) form.
 * Per (batch b, head h), token t:
 *   log f_t = log sigmoid(f~_t)            (sigmoid forget gate)
 *   log i_t = i~_t                         (exponential input gate)
 *   m_t     = max(log f_t + m_{t-1}, log i_t)
 *   C'_t    = exp(log f_t + m_{t-1} - m_t) C'_{t-1} + exp(i~_t - m_t) v_t k_t^T
 *   n'_t    = exp(log f_t + m_{t-1} - m_t) n'_{t-1} + exp(i~_t - m_t) k_t
 *   h_t     = sigmoid(o~_t) (.) (C'_t q_t) / max(|n'_t . q_t|, exp(-m_t))
 * The state is kept and returned stabilized: C' = C e^{-m}, n' = n e^{-m}.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, contiguous, row-major, in device memory, and owned by
 *     the caller.  The library allocates no device memory and keeps no mutable
 *     global state; calls on different streams are independent.
 *   - Layouts: q,k [B,NH,S,d_qk]; v [B,NH,S,d_v]; i_pre,f_pre [B,NH,S] fp32;
 *     o_pre [B,NH,S,d_v] fp32 (the output gate is applied component-wise);
 *     h_out [B,NH,S,d_v]; C [B,NH,d_v,d_qk] fp32 (row r of a head's C holds value
 *     dimension r); n [B,NH,d_qk] fp32; m [B,NH] fp32.
 *   - dtype gives the element type of q, k, v and h_out (fp32 or bf16); the gate
 *     pre-activations and the state are always fp32.
 *   - stream is a hipStream_t passed as void* (NULL = the default stream).  Calls
 *     enqueue work and return without synchronizing.
 *   - Errors: every argument is validated before anything is enqueued; on a bad
 *     argument nothing is launched and a status other than MLSTM_OK is returned.
 *     A failed launch returns MLSTM_ERR_HIP.  mlstm_error_detail() gives a
 *     human-readable reason for the last failure on the calling thread.  NaN or
 *     Inf in the inputs are propagated, not checked.
 *   - Outputs must not alias inputs (except where an entry point says "in place").
 *     mlstm_fwd_parallel, mlstm_fwd_parallel_state, mlstm_fwd_prepare,
 *     mlstm_fwd_scan and mlstm_step check it: a buffer they write (h_out, the
 *     final or in-place state, the workspace) that shares a byte with any other
 *     buffer of the call is rejected with MLSTM_ERR_INVALID_ARG.
 *   - Alignment: tensors the kernels access with vector loads or stores must be
 *     16-byte aligned (fwd: q, k, v, o_pre, h_out, C_final, n_final; step: q, k,
 *     C, n); every other pointer needs the alignment of its element type.
 */
#ifndef MLSTM_H
#define MLSTM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mlstm_status {
    MLSTM_OK = 0,
    MLSTM_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, bad chunk, ...  */
    MLSTM_ERR_UNSUPPORTED = 2,   /* valid but outside what the kernels implement     */
    MLSTM_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required       */
    MLSTM_ERR_HIP = 4            /* the HIP runtime reported an error                */
} mlstm_status;

typedef enum mlstm_dtype {
    MLSTM_F32 = 0,
    MLSTM_BF16 = 1
} mlstm_dtype;

/* activation of the sLSTM forget gate (slstm_fwd) */
typedef enum mlstm_forget_act {
    MLSTM_FORGET_SIGMOID = 0,    /* log f = log sigmoid(a_f) */
    MLSTM_FORGET_EXP = 1         /* log f = a_f              */
} mlstm_forget_act;

/* activation of the mLSTM block's external output gate (mlstm_block_epilogue) */
typedef enum mlstm_gate_act {
    MLSTM_GATE_SIGMOID = 0,      /* sigmoid(z)        */
    MLSTM_GATE_SWISH = 1         /* z * sigmoid(z)    */
} mlstm_gate_act;

/*
 * Bytes of device workspace a forward over these sizes needs (0 if none): what
 * mlstm_fwd_parallel (and its two stages) need when S is a multiple of chunk,
 * and what mlstm_fwd_parallel_state needs for any S >= 1.  Returns 0 as well for
 * arguments both would reject.
 */
size_t mlstm_fwd_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, int chunk,
                                 mlstm_dtype dtype);

/*
 * Chunkwise parallel forward over whole sequences (section 2.3, parallel form),
 * from the zero state C' = 0, n' = 0, m = 0.
 *
 * Tokens are processed in chunks of `chunk` tokens: inside a chunk the cell is
 * evaluated in its quadratic form with the log-forget cumulative-sum decay
 * matrix and a per-row stabilizer; the stabilized state (C', n', m) is carried
 * from chunk to chunk.  Results agree with the token-by-token recurrence up to
 * rounding for every chunk size.
 *
 * Where it runs: bf16 inputs with d_qk up to 1024 run on the matrix cores
 * (MFMA), in chunks of 64 tokens (also for chunk = 128, and for chunk = 16 or 32
 * except d_qk 128 and 384 at chunk 32, which have tilings of their own); when S
 * is not a multiple of that, the last S mod 64 tokens run on the vector-ALU
 * kernel.  The matrix-core tilings cover d_qk multiples of 64; any other d_qk
 * runs at the next multiple of 64 on copies of q and k (and of C_init, n_init)
 * padded with zero key columns, which change no product of the cell (section
 * 2.3: q and k enter only through contractions over the key dimension); the
 * final C' and n' are narrowed back to d_qk.  fp32 inputs and bf16 d_qk above
 * 1024 run entirely on the vector ALUs, which is correct at every size but two
 * to three orders of magnitude slower on wide heads (d_qk = 2048: about 0.7
 * TFLOP/s).  Only the matrix-core path uses the workspace; at (padded) d_qk 512
 * and 1024 it also holds copies of q and k in the order the matrix-core operands
 * are read (2 * B*NH*S*d_qk bf16 elements), and at a padded d_qk the padded
 * copies of q and k (2 * B*NH*S*d_pad bf16) and of the initial and final C'
 * and n' (2 * B*NH*(d_v + 1)*d_pad fp32).
 *
 * Arguments
 *   q, k, v         inputs, dtype, layouts above (read only)
 *   i_pre, f_pre    input / forget gate pre-activations [B,NH,S] fp32
 *   o_pre           output gate pre-activations [B,NH,S,d_v] fp32
 *   B, NH, S        batch, heads, tokens per sequence: all >= 1
 *   d_qk, d_v       key/query and value dimensions: multiples of 16, <= 4096
 *   chunk           16, 32, 64 or 128; S must be a multiple of chunk
 *   dtype           MLSTM_F32 or MLSTM_BF16
 *   h_out           [B,NH,S,d_v] dtype, written
 *   C_final, n_final, m_final
 *                   final stabilized state [B,NH,d_v,d_qk], [B,NH,d_qk], [B,NH]
 *                   fp32, written; the exact recurrent m_S is returned, so the
 *                   triple can be handed to mlstm_step to continue decoding
 *   workspace       device buffer of at least mlstm_fwd_workspace_bytes(...)
 *                   bytes (may be NULL when that is 0); its contents on entry
 *                   do not matter and are clobbered
 *   stream          hipStream_t or NULL
 */
mlstm_status mlstm_fwd_parallel(const void *q, const void *k, const void *v,
                                const float *i_pre, const float *f_pre, const float *o_pre,
                                int B, int NH, int S, int d_qk, int d_v, int chunk,
                                mlstm_dtype dtype,
                                void *h_out, float *C_final, float *n_final, float *m_final,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * mlstm_fwd_parallel for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, layouts, results and rules as mlstm_fwd_parallel, without the
 * workspace: the kernels use instead a scratch array the library holds in device
 * memory, one per GPU, of mlstm_fwd_noalloc_scratch_bytes() bytes (160 MiB),
 * kept from the first call on that GPU until the process ends.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine); the
 * first call on a device looks up that device's copy of the array once.
 *   - A forward whose workspace (mlstm_fwd_workspace_bytes) exceeds the scratch
 *     is rejected with MLSTM_ERR_UNSUPPORTED before anything is enqueued (the
 *     1.3B-class layer, B=4 NH=4 S=2048 d=1024, needs about 13 MB).
 *   - Every call on one GPU shares its array: calls that overlap in time on one
 *     GPU (two streams, or two threads) race and corrupt each other's results.
 *     Serialize them.  The scratch needs no clearing between calls (every byte
 *     the kernels read is written first by the same call).
 *   - The current HIP device must be the GPU the tensors and stream belong to.
 */
size_t mlstm_fwd_noalloc_scratch_bytes(void);
mlstm_status mlstm_fwd_parallel_noalloc(const void *q, const void *k, const void *v,
                                        const float *i_pre, const float *f_pre, const float *o_pre,
                                        int B, int NH, int S, int d_qk, int d_v, int chunk,
                                        mlstm_dtype dtype,
                                        void *h_out, float *C_final, float *n_final, float *m_final,
                                        void *stream);

/*
 * Chunkwise parallel forward that continues from a given stabilized state and
 * accepts any sequence length (section 2.3: the recurrence carried across the
 * chunks of the parallel form; a sequence split anywhere and run piece by piece,
 * each piece from the state the previous one returned, gives the result of one
 * run over the whole sequence, up to rounding).
 *
 * Same arguments, layouts and rules as mlstm_fwd_parallel, except:
 *   S               any length >= 1; when S is not a multiple of chunk, the
 *                   last S % chunk tokens form a shorter final chunk
 *   C_init, n_init, m_init
 *                   stabilized state entering token 0: [B,NH,d_v,d_qk],
 *                   [B,NH,d_qk], [B,NH] fp32, read only (C_init 16-byte aligned)
 *                   -- e.g. the final state of an earlier call, or of
 *                   mlstm_step.  All three NULL = the zero state.  Giving only
 *                   some of them is MLSTM_ERR_INVALID_ARG, and so is any
 *                   overlap between them and C_final, n_final, m_final (pass a
 *                   second buffer to continue a state).
 *   workspace       at least mlstm_fwd_workspace_bytes(B, NH, S, ...) bytes
 * With S a multiple of chunk and the zero state it computes exactly what
 * mlstm_fwd_parallel computes.
 */
mlstm_status mlstm_fwd_parallel_state(const void *q, const void *k, const void *v,
                                      const float *i_pre, const float *f_pre, const float *o_pre,
                                      int B, int NH, int S, int d_qk, int d_v, int chunk,
                                      mlstm_dtype dtype,
                                      const float *C_init, const float *n_init, const float *m_init,
                                      void *h_out, float *C_final, float *n_final, float *m_final,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * The two stages of mlstm_fwd_parallel, for callers that schedule them apart
 * (e.g. to time or overlap them).  Same arguments and rules as
 * mlstm_fwd_parallel; on one stream and with one workspace,
 *   mlstm_fwd_prepare(...) followed by mlstm_fwd_scan(...)
 * computes exactly what mlstm_fwd_parallel(...) computes.
 *   prepare: per chunk, in parallel over all chunks, the in-chunk cumulative log
 *            forget gate, the chunk-local stabilizer and the decayed intra-chunk
 *            scores, written to the workspace (a no-op for shapes whose
 *            forward runs as a single kernel)
 *   scan:    the sequential pass over chunks that carries (C', n', m) and writes
 *            h_out and the final state; reads what prepare left in the workspace
 */
mlstm_status mlstm_fwd_prepare(const void *q, const void *k,
                               const float *i_pre, const float *f_pre,
                               int B, int NH, int S, int d_qk, int d_v, int chunk,
                               mlstm_dtype dtype,
                               void *workspace, size_t workspace_bytes, void *stream);
mlstm_status mlstm_fwd_scan(const void *q, const void *k, const void *v,
                            const float *i_pre, const float *f_pre, const float *o_pre,
                            int B, int NH, int S, int d_qk, int d_v, int chunk,
                            mlstm_dtype dtype,
                            void *h_out, float *C_final, float *n_final, float *m_final,
                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * One-token recurrent decode step (section 2.3, the recurrence applied once).
 *
 * The stabilized state (C, n, m) is read and updated IN PLACE; each element is
 * read and rewritten by the same thread, so no separate output state exists.
 *   q, k            [B,NH,d_qk] dtype;  v [B,NH,d_v] dtype
 *   i_pre, f_pre    [B,NH] fp32;        o_pre [B,NH,d_v] fp32
 *   B, NH           >= 1;  d_qk, d_v multiples of 16, <= 4096
 *   C, n, m         [B,NH,d_v,d_qk], [B,NH,d_qk], [B,NH] fp32, in place
 *   h_out           [B,NH,d_v] dtype, written
 * The dot products n'.q and C'q are accumulated in fp64 over exactly the fp32
 * state values written back, so h_out is the retrieval from the returned state.
 */
mlstm_status mlstm_step(const void *q, const void *k, const void *v,
                        const float *i_pre, const float *f_pre, const float *o_pre,
                        int B, int NH, int d_qk, int d_v, mlstm_dtype dtype,
                        float *C, float *n, float *m, void *h_out, void *stream);

/*
 * Bytes of device workspace mlstm_bwd_parallel needs for these sizes (0 for
 * arguments it would reject).
 */
size_t mlstm_bwd_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, mlstm_dtype dtype);

/*
 * Gradients of the forward from the zero state (what mlstm_fwd_parallel computes
 * for h_out) with respect to all six inputs, given the gradient dh of a loss with
 * respect to h_out.  Section 2.3 (the parallel form of the cell, which is what is
 * differentiated) and section 2.2 (the stabilizer m_t changes no output, so no
 * gradient flows through it; the gradients are computed in the stabilized
 * quantities and are those of the unstabilized cell).
 *
 * With F_t the cumulative log forget gate and D_ts = exp(F_t - F_s + i~_s) for
 * s <= t, the forward is h_t = sigmoid(o~_t) (.) num_t / max(|den_t|, 1) with
 * num_t = sum_s D_ts (q_t . k_s) v_s and den_t = sum_s D_ts (q_t . k_s).  Where
 * the floor is active (|den_t| <= 1) den_t receives no gradient.
 *
 * Arguments
 *   q, k, v, i_pre, f_pre, o_pre
 *                   the forward's inputs, layouts and dtype as for the forward
 *                   (read only)
 *   dh              [B,NH,S,d_v] dtype, gradient with respect to h_out (read only)
 *   B, NH, S        >= 1; S need not be a multiple of anything
 *   d_qk, d_v       multiples of 16, <= 4096
 *   dtype           MLSTM_F32 or MLSTM_BF16 (of q, k, v and dh)
 *   grad_q, grad_k  [B,NH,S,d_qk] fp32, written
 *   grad_v          [B,NH,S,d_v] fp32, written
 *   grad_i, grad_f  [B,NH,S] fp32, written (gradients w.r.t. i_pre and f_pre)
 *   grad_o          [B,NH,S,d_v] fp32, written (gradient w.r.t. o_pre)
 *   workspace       device buffer of at least mlstm_bwd_workspace_bytes(...)
 *                   bytes, 16-byte aligned; contents on entry do not matter.
 *                   bf16 with a width above 384 and S <= 16384 holds the
 *                   causal score-shaped matrices: about 8 S_p^2 bytes per
 *                   head, S_p = S rounded up to 128.  Otherwise, from S = 1024
 *                   on (bf16, d_qk and d_v <= 512), the sums over earlier keys
 *                   are carried through the stabilized state at every
 *                   256-token boundary, which the workspace holds too: about
 *                   12 d_v d_qk bytes per boundary and head
 *   stream          hipStream_t or NULL
 * Every pointer must be 16-byte aligned except i_pre, f_pre, grad_i, grad_f
 * (4 bytes).  Outputs must not alias inputs, the workspace or each other.
 */
mlstm_status mlstm_bwd_parallel(const void *q, const void *k, const void *v,
                                const float *i_pre, const float *f_pre, const float *o_pre,
                                const void *dh,
                                int B, int NH, int S, int d_qk, int d_v, mlstm_dtype dtype,
                                float *grad_q, float *grad_k, float *grad_v,
                                float *grad_i, float *grad_f, float *grad_o,
                                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Epilogue of the mLSTM block ("xLSTM: Extended Long Short-Term Memory",
 * Figure 10 and its caption): the cell output is normalized by a GroupNorm with
 * one group per head (a LayerNorm over the head's d_v channels with a
 * per-channel scale and shift), the learnable skip input is added, and the sum is
 * gated component-wise by the external output gate.  Per (b, head, t):
 *   mu = mean_r h_r,  var = mean_r (h_r - mu)^2     (population variance)
 *   y_r = (gn_weight_r (h_r - mu) / sqrt(var + eps) + gn_bias_r
 *          + skip_weight_r x_r) * act(z_r)
 * The caption does not name the gate's activation; act selects sigmoid or swish.
 *
 * Arguments
 *   h               [B,NH,S,d_v] dtype, the cell output (e.g. h_out of a forward)
 *   x               [B,NH,S,d_v] dtype, the skip input of each head's channels
 *   z               [B,NH,S,d_v] dtype, external output gate pre-activations
 *   gn_weight, gn_bias, skip_weight
 *                   [NH,d_v] fp32 per-channel parameters (channel r of head hd at
 *                   hd*d_v + r)
 *   B, NH, S        >= 1;  d_v a multiple of 16, <= 4096
 *   eps             >= 0 (finite); a row with zero variance needs eps > 0
 *   act             MLSTM_GATE_SIGMOID or MLSTM_GATE_SWISH
 *   dtype           MLSTM_F32 or MLSTM_BF16 (of h, x, z and y_out)
 *   y_out           [B,NH,S,d_v] dtype, written; may be the same buffer as h, x
 *                   or z (each element is read before it is written, by the same
 *                   thread), but must not partly overlap any of them
 * All tensor pointers must be 16-byte aligned.
 */
mlstm_status mlstm_block_epilogue(const void *h, const void *x, const void *z,
                                  const float *gn_weight, const float *gn_bias,
                                  const float *skip_weight,
                                  int B, int NH, int S, int d_v, float eps,
                                  mlstm_gate_act act, mlstm_dtype dtype,
                                  void *y_out, void *stream);

/*
 * The zero-state chunkwise forward (mlstm_fwd_parallel) followed by the block
 * epilogue (mlstm_block_epilogue) in one call: y_out receives the epilogue of the
 * cell output h, and h itself is not returned.  ("xLSTM: Extended Long Short-Term
 * Memory", section 2.3 for the cell and Figure 10 with its caption for the
 * epilogue.)  Two ways to run it, selected by `fuse`:
 *   fuse = 1  where the forward runs whole on the matrix cores with one 64-column
 *             value tile per head and one key part (bf16, d_v <= 64, d_qk <= 128
 *             after padding to a multiple of 64, S a multiple of the executed
 *             chunk), the scan applies the epilogue to each row of h in registers
 *             (finishing a chunk's rows during the next chunk) and h never passes
 *             through HBM; other shapes run as with fuse = 0.
 *   fuse = 0  the forward writes h into the workspace and the epilogue kernel
 *             reads it back.
 * The fused rows add their normalization to the scan's sequential chunk loop, while
 * the epilogue kernel runs over the whole chip at the memory rate: on one MI355X,
 * B=8, NH=16, S=2048, d_qk=d_v=64 took 0.198 ms fused against 0.188 ms unfused, so
 * fuse = 1 is for callers that must save the 2 * |h| bytes of HBM traffic.  The
 * result is the same up to rounding either way (the fused path normalizes h
 * before its rounding to the output dtype).
 *
 * Arguments: those of mlstm_fwd_parallel (without h_out) and of
 * mlstm_block_epilogue (without h), and fuse (0 or 1); x, z, gn_weight, gn_bias,
 * skip_weight and y_out must be 16-byte aligned, and y_out must not overlap any
 * other buffer.
 * workspace: at least mlstm_fwd_block_workspace_bytes(..., fuse) bytes.
 * Errors: as mlstm_fwd_parallel and mlstm_block_epilogue; nothing is launched
 * on a bad argument.
 */
size_t mlstm_fwd_block_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, int chunk,
                                       mlstm_dtype dtype, int fuse);
mlstm_status mlstm_fwd_parallel_block(const void *q, const void *k, const void *v,
                                      const float *i_pre, const float *f_pre, const float *o_pre,
                                      const void *x, const void *z,
                                      const float *gn_weight, const float *gn_bias,
                                      const float *skip_weight,
                                      int B, int NH, int S, int d_qk, int d_v, int chunk,
                                      float eps, mlstm_gate_act act, mlstm_dtype dtype, int fuse,
                                      void *y_out, float *C_final, float *n_final, float *m_final,
                                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * sLSTM recurrence with block-diagonal memory mixing ("xLSTM: Extended Long
 * Short-Term Memory", section 2.2: exponential gating, the normalizer state that
 * sums the input gate times all later forget gates, the stabilizer state m_t, and
 * memory mixing through recurrent connections from the hidden state to the cell
 * input and to the gates, within each head but not across heads; section 2.1 for
 * the LSTM cell it extends).  The pages describe the equations in words; this is
 * their plainest reading.  Per (b, head), cell r, with the head's recurrent
 * matrices R_g (g = z, i, f, o) and a_g = x_pre_g + R_g h_{t-1}:
 *   log i = a_i;  log f = log sigmoid(a_f) or a_f (forget);
 *   m_t = max(log f + m_{t-1}, log i)
 *   c_t = exp(log f + m_{t-1} - m_t) c_{t-1} + exp(log i - m_t) tanh(a_z)
 *   n_t = exp(log f + m_{t-1} - m_t) n_{t-1} + exp(log i - m_t)
 *   h_t = sigmoid(a_o) c_t / n_t
 * (c, n are kept stabilized: the unstabilized states times exp(-m_t).)  The input
 * projections x_pre = W x + b are computed by the caller (a dense GEMM).
 *
 * Arguments
 *   x_pre           [B,NH,S,4,d_h] fp32, gate order z, i, f, o (read only)
 *   R               [NH,4,d_h,d_h] dtype; R[hd][g][r][j] weighs h_{t-1}[j] into gate
 *                   g of cell r (read only)
 *   B, NH, S        >= 1;  d_h a multiple of 16, <= 192 (bf16) or <= 128 (fp32)
 *   forget          MLSTM_FORGET_SIGMOID or MLSTM_FORGET_EXP
 *   dtype           MLSTM_F32 or MLSTM_BF16: element type of R and h_out (the
 *                   recurrent products run on bf16 MFMA; fp32 R is split into
 *                   two bf16 parts, h into two bf16 parts)
 *   c_init, n_init, m_init, h_init
 *                   [B,NH,d_h] fp32 state entering token 0, all four or none
 *                   (none = zero state, m = 0)
 *   h_out           [B,NH,S,d_h] dtype, written
 *   c_final, n_final, m_final, h_final
 *                   [B,NH,d_h] fp32, written; each may be the same buffer as the
 *                   matching initial one (in place), but no other overlap
 * x_pre and R must be 16-byte aligned, the state buffers 8-byte aligned, h_out
 * aligned to its element type.
 */
mlstm_status slstm_fwd(const float *x_pre, const void *R, int B, int NH, int S, int d_h,
                       mlstm_forget_act forget, mlstm_dtype dtype,
                       const float *c_init, const float *n_init, const float *m_init, const float *h_init,
                       void *h_out, float *c_final, float *n_final, float *m_final, float *h_final,
                       void *stream);

/* Static description of a status code. */
const char *mlstm_status_string(mlstm_status status);

/* Reason for the most recent failed call on this thread ("" if none). */
const char *mlstm_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* MLSTM_H */
