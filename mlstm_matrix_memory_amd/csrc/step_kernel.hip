// One-token recurrent decode step of the mLSTM cell ("xLSTM: Extended Long
// Short-Term Memory", section 2.3: covariance update eq. (18) with forget/input
// gates, normalizer with floor; section 2.2: stabilizer m_t).
//
// Bandwidth-bound: per head the stabilized memory C' (d_v x d_qk fp32) is read
// once and written once, in place; everything else is O(d).  One workgroup owns
// one (batch, head), so the in-place update of the per-head n' and m needs no
// cross-workgroup ordering: every thread reads m before the block barrier of the
// normalizer reduction, and m is written after it.
//
// Layout of the streaming loop: lane l of a wave covers the 16-byte column
// groups j = 4*l + 256*u (u < NJ) of a row, so one wave-wide load moves 1 KiB of
// a row with perfect coalescing; each wave walks rows r = wave, wave+W, ... with
// ROWS rows in flight per iteration to keep enough loads outstanding.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int STEP_THREADS = 512;
constexpr int STEP_WAVES = STEP_THREADS / 64;

// rows per wave per iteration: enough 16-byte loads in flight without spilling
template <int NJ> constexpr int step_rows() { return NJ <= 2 ? 4 : (NJ <= 4 ? 2 : 1); }

template <typename T, int NJ>
__global__ __launch_bounds__(STEP_THREADS) void step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ i_pre, const float* __restrict__ f_pre,
    const float* __restrict__ o_pre, int dqk, int dv,
    float* __restrict__ C, float* __restrict__ n, float* __restrict__ m, T* __restrict__ h)
{
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // s1: stabilized gates (every thread, redundantly; scalar gate math in fp64)
    const double log_f = log_sigmoid_f64((double)f_pre[bh]);
    const double log_i = (double)i_pre[bh];
    const double m_prev = (double)m[bh];
    const double m_t = fmax(log_f + m_prev, log_i);
    const float fs = exp_arg(log_f + m_prev - m_t);
    const float is = exp_arg(log_i - m_t);

    const T* qb = q + (size_t)bh * dqk;
    const T* kb = k + (size_t)bh * dqk;

    // s3: n' <- f' n' + i' k ; den = n' . q   (same thread reads and writes n'[j])
    // The two dot products of the step (n'.q here, C'q below) are accumulated in
    // fp64: when q is nearly orthogonal to a memory dominated by a few stored
    // pairs, both cancel, and fp32 accumulation error alone then exceeds the
    // fp32 path's tolerance.  The updated state elements themselves are fp32 (the
    // state's storage type), and the dot products are taken of exactly the values
    // stored, so h is the retrieval from the returned state.  The kernel is bound
    // by the state's HBM traffic; the fp64 arithmetic hides under it.
    __shared__ double red[STEP_WAVES];
    float* nb = n + (size_t)bh * dqk;
    double part = 0.0;
    for (int j = tid * 4; j < dqk; j += STEP_THREADS * 4) {
        f32x4 kk = load4(kb + j), qq = load4(qb + j);
        f32x4 nn = *reinterpret_cast<const f32x4*>(nb + j);
        nn = fs * nn + is * kk;
        *reinterpret_cast<f32x4*>(nb + j) = nn;
        part += (double)nn[0] * qq[0] + (double)nn[1] * qq[1] + (double)nn[2] * qq[2] + (double)nn[3] * qq[3];
    }
    part = wave_sum_f64(part);
    if (lane == 0) red[wave] = part;
    __syncthreads();  // all reads of m[bh] and n are done past this point
    double den = 0.0;
#pragma unroll
    for (int w = 0; w < STEP_WAVES; ++w) den += red[w];
    const double inv_denom = 1.0 / fmax(fabs(den), exp(-m_t));

    // this lane's key and query columns, kept in registers for all rows
    f32x4 kr[NJ], qr[NJ];
    bool ok[NJ];
#pragma unroll
    for (int u = 0; u < NJ; ++u) {
        const int j = 4 * lane + 256 * u;
        ok[u] = j < dqk;
        kr[u] = ok[u] ? load4(kb + j) : f32x4{0, 0, 0, 0};
        qr[u] = ok[u] ? load4(qb + j) : f32x4{0, 0, 0, 0};
    }

    // s2 + s4: stream the rows of C'
    constexpr int STEP_ROWS = step_rows<NJ>();
    float* Cb = C + (size_t)bh * dv * dqk;
    const T* vb = v + (size_t)bh * dv;
    const float* ob = o_pre + (size_t)bh * dv;
    T* hb = h + (size_t)bh * dv;
    for (int r0 = wave * STEP_ROWS; r0 < dv; r0 += STEP_WAVES * STEP_ROWS) {
        f32x4 c[STEP_ROWS][NJ];
#pragma unroll
        for (int rr = 0; rr < STEP_ROWS; ++rr) {
            const int r = r0 + rr;
#pragma unroll
            for (int u = 0; u < NJ; ++u) {
                const int j = 4 * lane + 256 * u;
                if (r < dv && ok[u])
                    c[rr][u] = __builtin_nontemporal_load(
                        reinterpret_cast<const f32x4*>(Cb + (size_t)r * dqk + j));
                else
                    c[rr][u] = f32x4{0, 0, 0, 0};
            }
        }
        double acc[STEP_ROWS];
#pragma unroll
        for (int rr = 0; rr < STEP_ROWS; ++rr) {
            const int r = r0 + rr;
            const float ivr = (r < dv) ? is * to_f32(vb[r]) : 0.0f;
            double a = 0.0;
#pragma unroll
            for (int u = 0; u < NJ; ++u) {
                f32x4 cn = fs * c[rr][u] + ivr * kr[u];
                c[rr][u] = cn;
                a += (double)cn[0] * qr[u][0] + (double)cn[1] * qr[u][1] + (double)cn[2] * qr[u][2] +
                     (double)cn[3] * qr[u][3];
            }
            acc[rr] = a;
        }
#pragma unroll
        for (int rr = 0; rr < STEP_ROWS; ++rr) {
            const int r = r0 + rr;
#pragma unroll
            for (int u = 0; u < NJ; ++u) {
                const int j = 4 * lane + 256 * u;
                if (r < dv && ok[u])
                    __builtin_nontemporal_store(c[rr][u],
                        reinterpret_cast<f32x4*>(Cb + (size_t)r * dqk + j));
            }
        }
#pragma unroll
        for (int rr = 0; rr < STEP_ROWS; ++rr) acc[rr] = wave_sum_f64(acc[rr]);
        if (lane < STEP_ROWS) {
            double mine = acc[0];
#pragma unroll
            for (int rr = 1; rr < STEP_ROWS; ++rr) if (lane == rr) mine = acc[rr];
            const int r = r0 + lane;
            if (r < dv) hb[r] = from_f32<T>(sigmoid(ob[r]) * (float)(mine * inv_denom));
        }
    }
    if (tid == 0) m[bh] = (float)m_t;
}

template <typename T, int NJ>
hipError_t launch_t(const StepArgs& a) {
    hipLaunchKernelGGL((step_kernel<T, NJ>), dim3(a.B * a.NH), dim3(STEP_THREADS), 0, a.stream,
                       (const T*)a.q, (const T*)a.k, (const T*)a.v, a.i_pre, a.f_pre, a.o_pre,
                       a.dqk, a.dv, a.C, a.n, a.m, (T*)a.h);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const StepArgs& a) {
    const int nj = (a.dqk + 255) / 256;
    if (nj <= 1) return launch_t<T, 1>(a);
    if (nj <= 2) return launch_t<T, 2>(a);
    if (nj <= 4) return launch_t<T, 4>(a);
    if (nj <= 8) return launch_t<T, 8>(a);
    return launch_t<T, 16>(a);
}

}  // namespace

hipError_t launch_step(const StepArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_dtype<bf16>(a);
    return launch_dtype<float>(a);
}

}  // namespace mlstm
