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
// workgroup runs one head for a tile of up to 4 sequences, all steps, with one
// wave per 16 cells (DHP / 16 waves):
//   - the wave holds the rows of all four gates of its 16 cells of the head's
//     recurrent matrices in registers, as bf16 MFMA A operands, for the whole
//     sequence (an fp32 matrix is held as bf16 hi + lo pairs);
//   - h_{t-1} of the tile sits in LDS as the B operand: columns s and s + 4 hold
//     bf16(h) of sequence s, columns s + 8 and s + 12 the remainder h - bf16(h),
//     so one 16-column MFMA gives R bf16(h) and R (h - bf16(h)) side by side, a
//     lane swap adds them (the split costs no extra MFMA), and every (cell,
//     sequence) pair of the wave has a lane of its own for the gate arithmetic;
//   - the four gate sums of a cell land in the same lanes, which keep that cell's
//     (c, n, m) for its sequence in registers and update it in place: no LDS
//     round trip for the gates;
//   - h goes to a second LDS buffer (ping-pong), so a step needs one barrier;
//   - the input pre-activations are loaded several steps ahead.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int SL_BT = 4;                   // sequences per workgroup

template <int DHP>
constexpr int sl_threads() { return 4 * DHP; }    // one wave per 16 cells

// steps of input pre-activations in flight (8 registers each), as many as the
// registers left beside the recurrent matrices allow
template <typename T, int DHP>
constexpr int sl_prefetch() { return DHP > 128 ? 2 : 4; }

// where lanes that own no cell store their (ignored) h, one 8-byte slot per lane,
// and read their input pre-activations (zeros, never written)
__device__ __align__(16) float slstm_sink[128];
__device__ __align__(16) float slstm_zero[8];

template <int DHP>
struct alignas(16) SlstmSmem {
    bf16 hb[2][16 * (DHP + 8)];            // ping-pong B operand: [column][cell], hi 0..7, lo 8..15
};

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

// gate math on the hardware exp / log / reciprocal (about 1 ulp each)
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_sigmoid(float x) { return fast_rcp(1.0f + __expf(-x)); }
__device__ __forceinline__ float fast_log_sigmoid(float x) { return fminf(x, 0.0f) - __logf(1.0f + __expf(-fabsf(x))); }
__device__ __forceinline__ float fast_tanh(float x) {
    const float e = __expf(-2.0f * fabsf(x));
    return copysignf((1.0f - e) * fast_rcp(1.0f + e), x);
}

// value of lane (l + 8) mod 16 of the same 16-lane row (DPP row rotate by 8, VALU only)
__device__ __forceinline__ float row_swap8(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// T: dtype of R and h_out.  DHP: d_h rounded up to 64, 128 or (bf16) 192.
// FEXP: forget gate exp (log f = a_f) instead of sigmoid.
//
// Lane layout of a wave (16 cells, rows 16 w + 4 g + i of each gate): after the
// products, lane l of 16-lane row g holds the bf16(h) (l % 16 < 8) or remainder
// (l % 16 >= 8) part of the four gate sums of cells 4g + i for sequence l % 4;
// lane l then updates cell 4g + (l % 16) / 4 of that sequence, taking the other
// part from lane l + 8 (mod 16), which holds it for the same sequence.
template <typename T, int DHP, bool FEXP>
__global__ __launch_bounds__(sl_threads<DHP>()) void slstm_kernel(
    const float* __restrict__ x_pre, const T* __restrict__ R, int B, int NH, int S, int dh,
    const float* __restrict__ c0, const float* __restrict__ n0, const float* __restrict__ m0,
    const float* __restrict__ h0, T* __restrict__ h, float* __restrict__ cF, float* __restrict__ nF,
    float* __restrict__ mF, float* __restrict__ hF)
{
    constexpr bool SPLIT = sizeof(T) == 4;             // fp32 R: hi + lo A operands
    constexpr int P = DHP + 8;
    constexpr int KS = DHP / 32;                       // k-steps over the cells
    __shared__ SlstmSmem<DHP> sm;

    const int hd = blockIdx.x % NH, b0 = (blockIdx.x / NH) * SL_BT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;
    const int ci = ln >> 2, bl = ln & 3;               // lane updates cell 4g + ci of sequence bl
    const int r0 = 16 * wave + 4 * g + ci;             // this lane's cell
    const int b = b0 + bl;
    const bool own = b < B && r0 < dh;                 // lane updates (and stores) these cells

    // rows of the four gates of this wave's 16 cells as A operands
    bf16x8 ra[4][KS], rl[SPLIT ? 4 : 1][SPLIT ? KS : 1];
    {
        const T* Rh = R + (size_t)hd * 4 * dh * dh;
        const int r = 16 * wave + ln;
#pragma unroll
        for (int gt = 0; gt < 4; ++gt)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                const int c = 32 * kk + 8 * g;
                bf16x8 hi, lo;
                load_r(Rh + ((size_t)gt * dh + r) * dh + c, r < dh && c < dh, hi, lo);
                ra[gt][kk] = hi;
                if constexpr (SPLIT) rl[gt][kk] = lo;
            }
    }

    for (int e = tid; e < 2 * 16 * P; e += sl_threads<DHP>()) (&sm.hb[0][0])[e] = (bf16)0.0f;
    __syncthreads();
    float cs = 0.0f, ns = 0.0f, ms = 0.0f, hv = 0.0f;
    const size_t st0 = ((size_t)b * NH + hd) * dh + r0;
    // h of sequence bl as bf16 hi (columns bl, bl + 4) and remainder (bl + 8, bl + 12)
    auto put_h = [&](bf16* hb, float x) {
        const bf16 hi = (bf16)x, lo = (bf16)(x - (float)hi);
        hb[bl * P + r0] = hi;
        hb[(bl + 4) * P + r0] = hi;
        hb[(bl + 8) * P + r0] = lo;
        hb[(bl + 12) * P + r0] = lo;
    };
    if (own && c0) {
        cs = c0[st0];
        ns = n0[st0];
        ms = m0[st0];
        hv = h0[st0];
        put_h(sm.hb[0], hv);
    }

    // Wait here for the matrix and state loads: inside the step loop the compiler
    // cannot tell them from the loads in flight across iterations and would wait
    // for every outstanding load before each step's first product.
    __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0), expcnt and lgkmcnt unconstrained

    // The step's input pre-activations (gate gt at x_pre[b][hd][t][gt][r0, r0+1])
    // are loaded PD steps ahead into a ring of registers (the step loop is unrolled
    // by PD so the ring index is static), so their memory latency hides behind PD
    // steps.  They are loaded unconditionally from a valid address -- lanes that own
    // no cell read zeros, steps past the end re-read the last -- so the loaded
    // registers carry into their step without a select (which would make the
    // compiler wait for them at once).
    constexpr int PD = sl_prefetch<T, DHP>();
    const float* xb = own ? x_pre + ((size_t)b * NH + hd) * S * 4 * dh + r0 : slstm_zero;
    const size_t xstep = own ? (size_t)4 * dh : 0;
    const int goff = own ? dh : 0;
    float xr[PD][4];
#pragma unroll
    for (int u = 0; u < PD; ++u)
#pragma unroll
        for (int gt = 0; gt < 4; ++gt) xr[u][gt] = xb[(size_t)min(u, S - 1) * xstep + gt * goff];
    // h of lanes that own no cell goes to a sink, so the store needs no branch
    T* hrow = own ? h + ((size_t)b * NH + hd) * S * dh + r0 : reinterpret_cast<T*>(slstm_sink) + lane;
    const size_t hstep = own ? (size_t)dh : 0;

    // One step; branch free, so that the compiler can count the loads in flight
    // (a branch around a load or store makes it wait for all of them).  Lanes that
    // own no cell compute on zero inputs: their values stay finite and only reach
    // cells and sequences that are not stored (padded cells meet zero matrix columns).
    // Gate arithmetic: with d = log f + m_{t-1} - log i, exactly one of the
    // stabilized gates is 1 and the other exp(-|d|); sigmoid(a_o) c / n takes one
    // reciprocal.
    auto step = [&](int t, float (&xu)[4]) __attribute__((always_inline)) {
        const int cur = t & 1;
        lds_barrier();                                 // h_{t-1} complete in hb[cur]; loads stay in flight
        f32x4 acc[4];
#pragma unroll
        for (int gt = 0; gt < 4; ++gt) acc[gt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 hbv = *reinterpret_cast<const bf16x8*>(sm.hb[cur] + ln * P + 32 * kk + 8 * g);
#pragma unroll
            for (int gt = 0; gt < 4; ++gt) {
                acc[gt] = mfma(ra[gt][kk], hbv, acc[gt]);
                if constexpr (SPLIT) acc[gt] = mfma(rl[gt][kk], hbv, acc[gt]);
            }
        }
        {
            // gate sums of cell 4g + ci: this lane's column of row ci, plus the partner
            // column (lane l + 8 mod 16, the other part of the same sequence) of the same
            // row, which the partner sends while receiving its own row ci ^ 2 from here
            float a[4];
#pragma unroll
            for (int gt = 0; gt < 4; ++gt) {
                const float mine = ci == 0 ? acc[gt][0] : ci == 1 ? acc[gt][1] : ci == 2 ? acc[gt][2] : acc[gt][3];
                const float send = ci == 0 ? acc[gt][2] : ci == 1 ? acc[gt][3] : ci == 2 ? acc[gt][0] : acc[gt][1];
                a[gt] = mine + row_swap8(send) + xu[gt];
            }
            const float lf = FEXP ? a[2] : fast_log_sigmoid(a[2]);
            const float d = lf + ms - a[1];
            const float e = __expf(-fabsf(d));
            const float fs = d >= 0.0f ? 1.0f : e, is = d >= 0.0f ? e : 1.0f;
            cs = fs * cs + is * fast_tanh(a[0]);
            ns = fs * ns + is;
            ms = fmaxf(lf + ms, a[1]);
            hv = cs * fast_rcp(ns * (1.0f + __expf(-a[3])));
        }
        hrow[(size_t)t * hstep] = from_f32<T>(hv);
        put_h(sm.hb[cur ^ 1], hv);
        const size_t tn = (size_t)min(t + PD, S - 1) * xstep;
#pragma unroll
        for (int gt = 0; gt < 4; ++gt) xu[gt] = xb[tn + gt * goff];
    };
    const int nfull = S - S % PD;
    for (int t0 = 0; t0 < nfull; t0 += PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) step(t0 + u, xr[u]);
    }
#pragma unroll
    for (int u = 0; u < PD; ++u)
        if (nfull + u < S) step(nfull + u, xr[u]);
    if (own) {
        cF[st0] = cs;
        nF[st0] = ns;
        mF[st0] = ms;
        hF[st0] = hv;
    }
}

template <typename T, bool FEXP>
hipError_t launch_slstm_t(const SlstmArgs& a) {
    const dim3 grid((unsigned)(a.NH * ((a.B + SL_BT - 1) / SL_BT)));
    const T* R = (const T*)a.R;
    T* h = (T*)a.h;
#define SL_CASE(D)                                                                                               \
    if (a.dh <= D) {                                                                                             \
        hipLaunchKernelGGL((slstm_kernel<T, D, FEXP>), grid, dim3(sl_threads<D>()), 0, a.stream, a.x_pre, R, a.B, \
                           a.NH, a.S, a.dh, a.c0, a.n0, a.m0, a.h0, h, a.c, a.n, a.m, a.hlast);                  \
        return hipGetLastError();                                                                                \
    }
    SL_CASE(64)
    SL_CASE(128)
    if constexpr (sizeof(T) == 2) { SL_CASE(192) }
#undef SL_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_slstm(const SlstmArgs& a) {
    if (a.dtype == MLSTM_BF16) return a.forget_exp ? launch_slstm_t<bf16, true>(a) : launch_slstm_t<bf16, false>(a);
    return a.forget_exp ? launch_slstm_t<float, true>(a) : launch_slstm_t<float, false>(a);
}

}  // namespace mlstm
