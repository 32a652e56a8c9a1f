// sLSTM recurrence with block-diagonal memory mixing ("xLSTM: Extended Long
// Short-Term Memory", section 2.2: exponential gating with normalizer and
// stabilizer states; memory mixing through recurrent connections from the hidden
// state to the cell input and the gates, within a head and not across heads).
//
// Per (b, head), cells r < d_h, gate pre-activations a = x_pre_t + R h_{t-1}
// (gates z, i, f, o; R_g of the head is d_h x d_h, row = output cell):
//   log i = a_i,  log f = log sigmoid(a_f) or a_f,  m_t = max(log f + m_{t-1}, log i)
//   c_t = e^{log f + m_{t-1} - m_t} c_{t-1} + e^{log i - m_t} tanh(a_z)
//   n_t = e^{log f + m_{t-1} - m_t} n_{t-1} + e^{log i - m_t}
//   h_t = sigmoid(a_o) c_t / n_t
//
// The recurrence is sequential in t, so a step's latency is what counts.  One
// workgroup runs one head for a tile of up to 8 sequences, all steps:
//   - the head's four recurrent matrices stay in registers for the whole sequence
//     as bf16 MFMA A operands (rows = 4 * DH gate rows, 16-row blocks dealt to the
//     waves; fp32 matrices are held as bf16 hi + lo pairs);
//   - h_{t-1} of the tile sits in LDS as the B operand: columns 0..7 hold bf16(h)
//     of the 8 sequences, columns 8..15 the rounding remainder h - bf16(h), so one
//     16-column MFMA gives R bf16(h) and R (h - bf16(h)) side by side and a lane
//     swap adds them (the split costs no extra MFMA);
//   - R h goes through LDS to the thread that owns the cell's (c, n, m); that
//     thread has loaded the step's input pre-activations of its cells while the
//     products ran, updates the state in fp32 registers, and writes h_t out and
//     back to LDS.
// Two workgroup barriers per step.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int SL_BT = 8;                   // sequences per workgroup

// threads per workgroup: 16 waves, or 8 at d_h 192, where a wave's share of the
// recurrent matrices needs more than the 128 registers a lane has at 16 waves
template <int DHP>
constexpr int sl_threads() { return DHP > 128 ? 512 : 1024; }

template <int DHP>
struct alignas(16) SlstmSmem {
    bf16 hb[16 * (DHP + 8)];               // B operand: [column][cell], hi columns 0..7, lo 8..15
    float gate[4 * DHP * SL_BT];           // [gate row][sequence]
};

__device__ __forceinline__ void store_h(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_h(bf16* p, float v) { *p = (bf16)v; }

// A operand (8 consecutive columns of one R row) from bf16 or fp32 memory
__device__ __forceinline__ void load_r(const bf16* p, bool ok, bf16x8& hi, bf16x8& lo) {
    hi = ok ? *reinterpret_cast<const bf16x8*>(p) : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    lo = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
}
__device__ __forceinline__ void load_r(const float* p, bool ok, bf16x8& hi, bf16x8& lo) {
    f32x4 a = ok ? load4(p) : f32x4{0, 0, 0, 0};
    f32x4 b = ok ? load4(p + 4) : f32x4{0, 0, 0, 0};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? a[e] : b[e - 4];
        hi[e] = (bf16)x;
        lo[e] = (bf16)(x - (float)hi[e]);
    }
}

// T: dtype of R and h_out.  DHP: d_h rounded up to 64, 128 or (bf16) 192.
template <typename T, int DHP>
__global__ __launch_bounds__(sl_threads<DHP>()) void slstm_kernel(
    const float* __restrict__ x_pre, const T* __restrict__ R, int B, int NH, int S, int dh, int forget_exp,
    const float* __restrict__ c0, const float* __restrict__ n0, const float* __restrict__ m0,
    const float* __restrict__ h0, T* __restrict__ h, float* __restrict__ cF, float* __restrict__ nF,
    float* __restrict__ mF, float* __restrict__ hF)
{
    constexpr int SL_THREADS = sl_threads<DHP>();
    constexpr int SL_WAVES = SL_THREADS / 64;
    constexpr bool SPLIT = sizeof(T) == 4;             // fp32 R: hi + lo A operands
    constexpr int P = DHP + 8;
    constexpr int RB = 4 * DHP / 16 / SL_WAVES;        // 16-row blocks per wave
    constexpr int KS = DHP / 32;                       // k-steps over the cells
    constexpr int NITEM = DHP * SL_BT;                 // (sequence, cell) pairs of the tile
    constexpr int IPT = (NITEM + SL_THREADS - 1) / SL_THREADS;
    __shared__ SlstmSmem<DHP> sm;

    const int hd = blockIdx.x % NH, b0 = (blockIdx.x / NH) * SL_BT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;

    // recurrent matrices of this head as A operands
    bf16x8 ra[RB][KS], rl[SPLIT ? RB : 1][SPLIT ? KS : 1];
    const T* Rh = R + (size_t)hd * 4 * dh * dh;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int row = 16 * (wave * RB + rb) + ln;    // gate row in the padded layout
        const int gate = row / DHP, r = row % DHP;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int c = 32 * kk + 8 * g;
            bf16x8 hi, lo;
            load_r(Rh + ((size_t)gate * dh + r) * dh + c, r < dh && c < dh, hi, lo);
            ra[rb][kk] = hi;
            if constexpr (SPLIT) rl[rb][kk] = lo;
        }
    }

    // state of the cells this thread updates: item = tid + SL_THREADS * j -> (sequence, cell)
    float cs[IPT], ns[IPT], ms[IPT];
    for (int e = tid; e < 16 * P; e += SL_THREADS) sm.hb[e] = (bf16)0.0f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int item = tid + SL_THREADS * j;
        const int bb = item / DHP, r = item % DHP, b = b0 + bb;
        cs[j] = ns[j] = ms[j] = 0.0f;
        if (item < NITEM && r < dh && b < B) {
            const size_t st = ((size_t)b * NH + hd) * dh + r;
            float hv = 0.0f;
            if (c0) { cs[j] = c0[st]; ns[j] = n0[st]; ms[j] = m0[st]; hv = h0[st]; }
            const bf16 hi = (bf16)hv;
            sm.hb[bb * P + r] = hi;
            sm.hb[(SL_BT + bb) * P + r] = (bf16)(hv - (float)hi);
        }
    }

    for (int t = 0; t < S; ++t) {
        // this step's input pre-activations of the thread's cells: issued before the
        // barrier and the products, used after them
        float xz[IPT], xi[IPT], xf[IPT], xo[IPT];
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int item = tid + SL_THREADS * j;
            const int bb = item / DHP, r = item % DHP, b = b0 + bb;
            xz[j] = xi[j] = xf[j] = xo[j] = 0.0f;
            if (item < NITEM && r < dh && b < B) {
                const float* xp = x_pre + (((size_t)b * NH + hd) * S + t) * 4 * dh + r;
                xz[j] = xp[0];
                xi[j] = xp[dh];
                xf[j] = xp[2 * dh];
                xo[j] = xp[3 * dh];
            }
        }
        __syncthreads();                               // h_{t-1} in LDS
        f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 hbv = *reinterpret_cast<const bf16x8*>(sm.hb + ln * P + 32 * kk + 8 * g);
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                acc[rb] = mfma(ra[rb][kk], hbv, acc[rb]);
                if constexpr (SPLIT) acc[rb] = mfma(rl[rb][kk], hbv, acc[rb]);
            }
        }
        // column ln + 8 holds R (h - bf16(h)) of sequence ln: add it in
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rb][i] += __shfl_xor(acc[rb][i], 8, 64);
            if (ln < SL_BT) {
                const int row = 16 * (wave * RB + rb) + 4 * g;
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.gate[(row + i) * SL_BT + ln] = acc[rb][i];
            }
        }
        __syncthreads();                               // gate pre-activations complete
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            const int item = tid + SL_THREADS * j;
            const int bb = item / DHP, r = item % DHP, b = b0 + bb;
            if (item < NITEM && r < dh && b < B) {
                const float az = sm.gate[(0 * DHP + r) * SL_BT + bb] + xz[j];
                const float ai = sm.gate[(1 * DHP + r) * SL_BT + bb] + xi[j];
                const float af = sm.gate[(2 * DHP + r) * SL_BT + bb] + xf[j];
                const float ao = sm.gate[(3 * DHP + r) * SL_BT + bb] + xo[j];
                const float lf = forget_exp ? af : log_sigmoid(af);
                const float mt = fmaxf(lf + ms[j], ai);
                const float fs = expf(lf + ms[j] - mt), is = expf(ai - mt);
                cs[j] = fs * cs[j] + is * tanhf(az);
                ns[j] = fs * ns[j] + is;
                ms[j] = mt;
                const float hv = sigmoid(ao) * cs[j] / ns[j];
                store_h(h + (((size_t)b * NH + hd) * S + t) * dh + r, hv);
                const bf16 hi = (bf16)hv;
                sm.hb[bb * P + r] = hi;
                sm.hb[(SL_BT + bb) * P + r] = (bf16)(hv - (float)hi);
            }
        }
    }
    // final state
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        const int item = tid + SL_THREADS * j;
        const int bb = item / DHP, r = item % DHP, b = b0 + bb;
        if (item < NITEM && r < dh && b < B) {
            const size_t st = ((size_t)b * NH + hd) * dh + r;
            cF[st] = cs[j];
            nF[st] = ns[j];
            mF[st] = ms[j];
            hF[st] = (float)sm.hb[bb * P + r] + (float)sm.hb[(SL_BT + bb) * P + r];
        }
    }
}

template <typename T>
hipError_t launch_slstm_t(const SlstmArgs& a) {
    const dim3 grid((unsigned)(a.NH * ((a.B + SL_BT - 1) / SL_BT)));
    const T* R = (const T*)a.R;
    T* h = (T*)a.h;
#define SL_CASE(D)                                                                                           \
    if (a.dh <= D) {                                                                                         \
        hipLaunchKernelGGL((slstm_kernel<T, D>), grid, dim3(sl_threads<D>()), 0, a.stream, a.x_pre, R, a.B, a.NH, \
                           a.S, a.dh, a.forget_exp, a.c0, a.n0, a.m0, a.h0, h, a.c, a.n, a.m, a.hlast);     \
        return hipGetLastError();                                                                            \
    }
    SL_CASE(64)
    SL_CASE(128)
    if constexpr (sizeof(T) == 2) { SL_CASE(192) }
#undef SL_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_slstm(const SlstmArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_slstm_t<bf16>(a);
    return launch_slstm_t<float>(a);
}

}  // namespace mlstm
