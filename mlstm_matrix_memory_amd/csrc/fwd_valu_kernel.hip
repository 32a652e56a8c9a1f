// Chunkwise parallel forward of the mLSTM cell on the vector ALUs (fp32 math).
// Also the tail kernel of a sequence whose length is not a multiple of the
// chunk: the last chunk simply has fewer tokens.
//
// "xLSTM: Extended Long Short-Term Memory": section 2.3 (covariance update
// eq. (18), normalizer with floor, parallel form of the recurrence), section 2.2
// (stabilizer m_t, eq. (17)).  This kernel serves the fp32 path and every shape
// the bf16 MFMA kernel does not cover.  It is exact up to fp32 rounding.
//
// Chunkwise form used here, per head, for a chunk of Lc tokens entering with the
// stabilized state (C', n', m_p):
//   b_tau   = sum_{j<=tau} log sigmoid(f~_j)            (in-chunk cumulative sum)
//   logD    = b_tau - b_s + i~_s  for s <= tau          (decay matrix, log domain)
//   m_tau   = max(b_tau + m_p, max_s logD_tau,s)        (= the recurrent m_t)
//   P       = (q_tau . k_s) exp(logD - m_tau),   a_tau = exp(b_tau + m_p - m_tau)
//   num     = P V + a (.) (Q C'^T),   den = rowsum(P) + a (.) (Q n')
//   h_tau   = sigmoid(o~_tau) (.) num / max(|den|, exp(-m_tau))
//   w_s     = exp(b_L - b_s + i~_s - m_L),   alpha = exp(b_L + m_p - m_L)
//   C'     <- alpha C' + V^T (w (.) K),   n' <- alpha n' + K^T w,   m_p <- m_L
// Every exponent above is <= 0, so nothing overflows however large i~ gets.
//
// Work split: grid (value tiles of TV rows, B*NH).  A workgroup owns TV rows of
// its head's C' and keeps them in the C_final buffer (each row has exactly one
// owner); the n' of the head is kept in LDS by every workgroup of the head and
// written back by tile 0.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int VALU_THREADS = 256;
constexpr int VALU_TV = 16;

template <typename T, int L>
__global__ __launch_bounds__(VALU_THREADS) void fwd_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ i_pre, const float* __restrict__ f_pre,
    const float* __restrict__ o_pre, int S, int Sx, int t_begin, int dqk, int dv,
    const float* __restrict__ C0, const float* __restrict__ n0, const float* __restrict__ m0,
    T* __restrict__ h, float* __restrict__ C, float* __restrict__ n, float* __restrict__ m)
{
    __shared__ float P[L][L + 1];
    __shared__ double sb[L], smd[L];              // cumulative log forget gate, stabilizer (fp64)
    __shared__ float si[L], sa[L], sw[L], sden[L], sfl[L];
    extern __shared__ float nq[];  // n' of this head, dqk floats

    const int vt = blockIdx.x;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int r_begin = vt * VALU_TV;
    const int rows = min(VALU_TV, dv - r_begin);

    // per-token tensors have Sx tokens per head; tokens [t_begin, S) are processed
    const T* qh = q + (size_t)bh * Sx * dqk;
    const T* kh = k + (size_t)bh * Sx * dqk;
    const T* vh = v + (size_t)bh * Sx * dv;
    const float* ih = i_pre + (size_t)bh * Sx;
    const float* fh = f_pre + (size_t)bh * Sx;
    const float* oh = o_pre + (size_t)bh * Sx * dv;
    T* hh = h + (size_t)bh * Sx * dv;
    float* Ch = C + (size_t)bh * dv * dqk + (size_t)r_begin * dqk;

    // initial state
    for (int idx = tid; idx < rows * dqk; idx += VALU_THREADS)
        Ch[idx] = C0 ? C0[(size_t)bh * dv * dqk + (size_t)r_begin * dqk + idx] : 0.0f;
    for (int j = tid; j < dqk; j += VALU_THREADS)
        nq[j] = n0 ? n0[(size_t)bh * dqk + j] : 0.0f;
    double m_prev = m0 ? (double)m0[bh] : 0.0;
    __syncthreads();

    for (int t0 = t_begin; t0 < S; t0 += L) {
        const int Lc = min(L, S - t0);
        // gates: log forget gate and its in-chunk cumulative sum
        if (tid < Lc) {
            sb[tid] = log_sigmoid_f64((double)fh[t0 + tid]);
            si[tid] = ih[t0 + tid];
        }
        __syncthreads();
        if (tid == 0) {
            double acc = 0.0;
            for (int s = 0; s < Lc; ++s) { acc += sb[s]; sb[s] = acc; }
        }
        // raw scores q_tau . k_s on and below the diagonal
        for (int idx = tid; idx < Lc * Lc; idx += VALU_THREADS) {
            const int tau = idx / Lc, s = idx % Lc;
            float dot = 0.0f;
            if (s <= tau) {
                const T* qr = qh + (size_t)(t0 + tau) * dqk;
                const T* kr = kh + (size_t)(t0 + s) * dqk;
                for (int j = 0; j < dqk; ++j) dot += to_f32(qr[j]) * to_f32(kr[j]);
            }
            P[tau][s] = dot;
        }
        __syncthreads();
        // per-row stabilizer and inter-chunk weight
        if (tid < Lc) {
            const int tau = tid;
            double mx = sb[tau] + m_prev;
            for (int s = 0; s <= tau; ++s) mx = fmax(mx, sb[tau] - sb[s] + (double)si[s]);
            smd[tau] = mx;
            sa[tau] = exp_arg(sb[tau] + m_prev - mx);
            sfl[tau] = exp_arg(-mx);
        }
        __syncthreads();
        for (int idx = tid; idx < Lc * Lc; idx += VALU_THREADS) {
            const int tau = idx / Lc, s = idx % Lc;
            if (s <= tau) P[tau][s] *= exp_arg(sb[tau] - sb[s] + (double)si[s] - smd[tau]);
        }
        __syncthreads();
        // normalizer: intra-chunk row sum + inter-chunk q . n'
        if (tid < Lc) {
            const int tau = tid;
            float intra = 0.0f;
            for (int s = 0; s <= tau; ++s) intra += P[tau][s];
            const T* qr = qh + (size_t)(t0 + tau) * dqk;
            float inter = 0.0f;
            for (int j = 0; j < dqk; ++j) inter += to_f32(qr[j]) * nq[j];
            sden[tau] = intra + sa[tau] * inter;
        }
        __syncthreads();
        // outputs of this tile's value rows
        for (int idx = tid; idx < Lc * rows; idx += VALU_THREADS) {
            const int tau = idx / rows, rr = idx % rows, r = r_begin + rr;
            float intra = 0.0f;
            for (int s = 0; s <= tau; ++s) intra += P[tau][s] * to_f32(vh[(size_t)(t0 + s) * dv + r]);
            const T* qr = qh + (size_t)(t0 + tau) * dqk;
            const float* cr = Ch + (size_t)rr * dqk;
            float inter = 0.0f;
            for (int j = 0; j < dqk; ++j) inter += to_f32(qr[j]) * cr[j];
            const float num = intra + sa[tau] * inter;
            const float denom = fmaxf(fabsf(sden[tau]), sfl[tau]);
            const size_t o = (size_t)(t0 + tau) * dv + r;
            hh[o] = from_f32<T>(sigmoid(oh[o]) * num / denom);
        }
        __syncthreads();
        // state update
        const double m_last = smd[Lc - 1];
        const double b_last = sb[Lc - 1];
        const float alpha = exp_arg(b_last + m_prev - m_last);
        if (tid < Lc) sw[tid] = exp_arg(b_last - sb[tid] + (double)si[tid] - m_last);
        __syncthreads();
        for (int idx = tid; idx < rows * dqk; idx += VALU_THREADS) {
            const int rr = idx / dqk, j = idx % dqk, r = r_begin + rr;
            float acc = 0.0f;
            for (int s = 0; s < Lc; ++s)
                acc += sw[s] * to_f32(vh[(size_t)(t0 + s) * dv + r]) * to_f32(kh[(size_t)(t0 + s) * dqk + j]);
            Ch[idx] = alpha * Ch[idx] + acc;
        }
        for (int j = tid; j < dqk; j += VALU_THREADS) {
            float acc = 0.0f;
            for (int s = 0; s < Lc; ++s) acc += sw[s] * to_f32(kh[(size_t)(t0 + s) * dqk + j]);
            nq[j] = alpha * nq[j] + acc;
        }
        m_prev = m_last;
        __syncthreads();
    }
    if (vt == 0) {
        for (int j = tid; j < dqk; j += VALU_THREADS) n[(size_t)bh * dqk + j] = nq[j];
        if (tid == 0) m[bh] = (float)m_prev;
    }
}

template <typename T, int L>
hipError_t launch_tl(const FwdArgs& a) {
    dim3 grid((a.dv + VALU_TV - 1) / VALU_TV, a.B * a.NH);
    hipLaunchKernelGGL((fwd_valu_kernel<T, L>), grid, dim3(VALU_THREADS), a.dqk * sizeof(float), a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.i_pre, a.f_pre, a.o_pre,
                       a.S, a.Sx, a.t_begin, a.dqk, a.dv, a.C0, a.n0, a.m0, (T*)a.h, a.C, a.n, a.m);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a) {
    switch (a.chunk) {
        case 16: return launch_tl<T, 16>(a);
        case 32: return launch_tl<T, 32>(a);
        case 64: return launch_tl<T, 64>(a);
        default: return launch_tl<T, 128>(a);
    }
}

}  // namespace

size_t valu_fwd_workspace_bytes(const FwdArgs&) { return 0; }

hipError_t launch_fwd_valu(const FwdArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_t<bf16>(a);
    return launch_t<float>(a);
}

}  // namespace mlstm
