// Internal declarations and device helpers of libmlstm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/mlstm.h"

namespace mlstm {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---- element conversions -------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// four consecutive elements starting at p (p 8- or 16-byte aligned)
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
    bf16x4 b = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)b[0], (float)b[1], (float)b[2], (float)b[3]};
}

// ---- gate math (fp32) ----------------------------------------------------
// log sigmoid(x) = min(x,0) - log(1 + exp(-|x|)), finite for every finite x
__device__ __forceinline__ float log_sigmoid(float x) {
    return fminf(x, 0.0f) - log1pf(expf(-fabsf(x)));
}
__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// The stabilizer and the exponent arguments of the gate weights are differences of
// running sums that reach O(100) in magnitude.  The normalized retrieval can cancel
// to a few parts in 1e4 in its denominator, so an absolute exponent error of 1e-6
// (fp32 rounding at that magnitude) already shows up at the percent level.  All
// scalar gate arithmetic is therefore done in fp64; only the final exp, applied to
// an accurate argument, is taken in fp32.
__device__ __forceinline__ double log_sigmoid_f64(double x) {
    return fmin(x, 0.0) - log1p(exp(-fabs(x)));
}
__device__ __forceinline__ float exp_arg(double x) { return expf((float)x); }

// ---- wavefront helpers (64 lanes) ------------------------------------------
// Index of the calling wave in its workgroup as a wave-uniform (scalar) value:
// branches and addresses that depend only on it then compile to scalar code,
// not to per-lane exec-mask manipulation.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// ---- MFMA helpers (v_mfma_f32_16x16x32_bf16) --------------------------------
// D[m][n] += sum_k A[m][k] B[k][n] over a 16 x 16 x 32 block.  Lane l supplies
// A[l%16][8(l/16) .. 8(l/16)+7] and B[8(l/16) .. +7][l%16] and holds
// D[4(l/16) + i][l%16], i = 0..3.  Which contraction index sits in which of the
// 32 k-slots is free, as long as A and B agree.
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// transposing LDS read (ds_read_b64_tr_b16): the 16 lanes of a group point at 4
// rows (lanes 4r .. 4r+3 at row r, 4 consecutive columns each); lane j receives
// column j of those 4 rows, in row order
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Workgroup barrier that orders LDS traffic only: this wave's LDS operations are
// complete (lgkmcnt 0) before it signals, but global loads and stores still in
// flight stay in flight, so register prefetches issued before the barrier keep
// overlapping with the work after it.  (The full __syncthreads fence would wait for
// them.)  The memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---- launchers (return hipSuccess or the launch error) --------------------
struct FwdArgs {
    const void* q; const void* k; const void* v;
    const float* i_pre; const float* f_pre; const float* o_pre;
    int B, NH, S, dqk, dv, chunk;
    int Sx;                 // token stride of the caller's per-token tensors (>= S)
    int t_begin;            // first token processed (fp32 / tail kernel); tokens [t_begin, S)
    mlstm_dtype dtype;
    void* h; float* C; float* n; float* m;
    const float* C0; const float* n0; const float* m0;   // initial state, all null = zero
    void* ws; size_t ws_bytes;
    hipStream_t stream;
    // block epilogue applied to h in the scan's output rows (mlstm_fwd_parallel_block
    // on a fusable shape; ep_x null = h is written as is): h then receives y
    const void* ep_x; const void* ep_z;
    const float* ep_gw; const float* ep_gb; const float* ep_sw;
    float ep_eps; int ep_act;
};

struct StepArgs {
    const void* q; const void* k; const void* v;
    const float* i_pre; const float* f_pre; const float* o_pre;
    int B, NH, dqk, dv;
    mlstm_dtype dtype;
    float* C; float* n; float* m; void* h;
    hipStream_t stream;
};

struct BwdArgs {
    const void* q; const void* k; const void* v; const void* dh;
    const float* i_pre; const float* f_pre; const float* o_pre;
    int B, NH, S, dqk, dv;
    mlstm_dtype dtype;
    float* dq; float* dk; float* dvv; float* di; float* df; float* dout;
    void* ws;
    hipStream_t stream;
};

struct EpilogueArgs {
    const void* h; const void* x; const void* z;
    const float* gn_w; const float* gn_b; const float* skip_w;
    int B, NH, S, dv;
    float eps;
    int act;                 // 0 sigmoid, 1 swish
    mlstm_dtype dtype;
    void* y;
    hipStream_t stream;
};

hipError_t launch_epilogue(const EpilogueArgs& a);

struct SlstmArgs {
    const float* x_pre; const void* R;
    int B, NH, S, dh;
    int forget_exp;          // 0: log f = log sigmoid(a_f); 1: log f = a_f
    mlstm_dtype dtype;       // of R and h
    const float* c0; const float* n0; const float* m0; const float* h0;   // all null = zero state
    void* h; float* c; float* n; float* m; float* hlast;
    hipStream_t stream;
};

hipError_t launch_slstm(const SlstmArgs& a);

hipError_t launch_step(const StepArgs& a);

// generic chunkwise forward on the vector ALUs (any supported shape, fp32 or bf16)
size_t valu_fwd_workspace_bytes(const FwdArgs& a);
hipError_t launch_fwd_valu(const FwdArgs& a);

// chunkwise forward on bf16 MFMA (bf16 inputs, shapes it supports)
int mfma_fwd_chunk(const FwdArgs& a);          // chunk the MFMA path executes for these widths, 0 = none
bool mfma_fwd_supported(const FwdArgs& a);
size_t mfma_fwd_workspace_bytes(const FwdArgs& a);
// whether the scan can apply the block epilogue to whole rows itself: the pipelined
// form with one value tile per head (d_v <= its 64-column tile)
bool mfma_fwd_block_fusable(const FwdArgs& a);
hipError_t launch_fwd_mfma_prepare(const FwdArgs& a);
hipError_t launch_fwd_mfma_scan(const FwdArgs& a);

// Row-major rows of src_row_bytes copied to rows of dst_row_bytes: zero-filled
// past the source width when widening, cut when narrowing (16-byte units where
// both widths and both pointers allow, else 4-byte units)
hipError_t launch_copy_cols(const void* src, void* dst, size_t rows, size_t src_row_bytes, size_t dst_row_bytes,
                            hipStream_t stream);

// backward of the zero-state forward (tiled quadratic form on the vector ALUs)
size_t bwd_workspace_bytes(const BwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

}  // namespace mlstm
