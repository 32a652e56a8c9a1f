// Chunkwise parallel forward of the mLSTM cell on bf16 MFMA (gfx950).
//
// "xLSTM: Extended Long Short-Term Memory": section 2.3 (covariance update
// eq. (18), normalizer with floor, multi-head independence and the parallel form
// of the recurrence) and section 2.2 (stabilizer m_t, eq. (17)).
//
// Two kernels, both on bf16 MFMA with fp32 accumulation:
//
// 1. chunk_prep (one workgroup per (head, chunk), all chunks in parallel)
//      b_tau     = in-chunk cumulative sum of log sigmoid(f~)
//      m_loc_tau = b_tau + max_{s<=tau}(i~_s - b_s)          chunk-local row max
//      P_loc     = (Q K^T) (.) exp(b_tau - b_s + i~_s - m_loc_tau)   (s <= tau)
//      den_loc   = rowsum(P_loc) (fp32),  w_loc_s = exp(b_L - b_s + i~_s - m_loc_L)
//    P_loc is stored in bf16 (it is the MFMA operand of the next kernel); every
//    exponent is <= 0 so nothing overflows.
//
// 2. chunk_scan (one workgroup per (head, tile of TV value columns), sequential
//    over the chunks of the head, state carried in MFMA accumulators)
//      m_tau = max(b_tau + m_p, m_loc_tau)   a_tau = exp(b_tau + m_p - m_tau)
//      r_tau = exp(m_loc_tau - m_tau)        (the exact recurrent stabilizer)
//      num   = r (.) (P_loc V) + a (.) (Q C'^T),  den = r (.) den_loc + a (.) (Q n')
//      h     = sigmoid(o~) (.) num / max(|den|, exp(-m_tau))
//      C'^T <- alpha C'^T + K^T (w (.) V),  n' <- alpha n' + K^T w,  m_p <- m_L
//      with w_s = exp(m_loc_L - m_L) w_loc_s and alpha = exp(b_L + m_p - m_L).
//
// Data movement of chunk_scan.  A wave owns 16 value columns and DQ/NK key rows
// of C'^T (fp32, D-layout of v_mfma_f32_16x16x32_bf16: lane l holds rows
// 4*(l/16)+i, column l%16 of each 16x16 block).  Per chunk the workgroup stages
// in LDS the chunk's P_loc, its V tile and w (.) V, then walks the key dimension
// in slabs of NK*SB columns of Q and K.  Products that contract the token axis
// (P V and K^T (w V)) need token-contiguous operands: they are read from the
// token-major LDS tiles with the gfx950 transposing read ds_read_b64_tr_b16
// (within a 16-lane group, lane j receives column j of the 4 rows the group's
// lanes point at).  Q C'^T contracts the key axis: its B operand is the state
// itself, converted to bf16 in registers, and Q is read so that each lane's 8 key
// indices match the 8 accumulator rows it holds.  LDS row pitches are chosen so
// every one of these reads is bank-conflict free.
//
// Precision.  q, k and v are exact bf16 inputs, but three MFMA operands carry
// computed fp32 values: P_loc, the state C' and w (.) V.  The retrieval divides
// by |n'^T q|, which is small exactly where q.k cancels, and there a single bf16
// rounding of those operands (relative 2^-9 per element) is amplified far past
// the tolerance.  Each of the three is therefore split as x = hi + lo with
// hi = bf16(x), lo = bf16(x - hi) (about 2^-17 relative together) and its
// product is taken as two MFMAs sharing the exact operand.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// transposing LDS read: 4 bf16 from the rows the lanes of this lane's 16-group point at
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 cvt8(f32x4 a, f32x4 b) {
    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

// inclusive scans over the lanes of one wave (64 lanes), fp64
__device__ __forceinline__ double wave_scan_add(double x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        double y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}
__device__ __forceinline__ double wave_scan_max(double x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        double y = __shfl_up(x, off, 64);
        if (lane >= off) x = fmax(x, y);
    }
    return x;
}

// ---------------------------------------------------------------------------
// workspace layout: P_loc as bf16 hi/lo pairs [heads][chunk][2][L][L]; the
// in-chunk cumulative log forget gate and chunk-local stabilizer as fp64
// [heads][S]; den_loc and w_loc as fp32 [heads][S]
// ---------------------------------------------------------------------------
struct Ws {
    bf16* P; double* b; double* mloc; float* den; float* wloc;
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline Ws ws_layout(void* base, size_t heads, size_t S, int L) {
    char* p = (char*)base;
    Ws w;
    w.P = (bf16*)p;                       p += align256(2 * heads * S * L * sizeof(bf16));
    w.b = (double*)p;                     p += align256(heads * S * sizeof(double));
    w.mloc = (double*)p;                  p += align256(heads * S * sizeof(double));
    w.den = (float*)p;                    p += align256(heads * S * sizeof(float));
    w.wloc = (float*)p;
    return w;
}
inline size_t ws_bytes(size_t heads, size_t S, int L) {
    return align256(2 * heads * S * L * sizeof(bf16)) + 2 * align256(heads * S * sizeof(double)) +
           2 * align256(heads * S * sizeof(float));
}

// ---------------------------------------------------------------------------
// kernel 1: per-chunk gates and intra-chunk decayed scores
// ---------------------------------------------------------------------------
constexpr int PREP_THREADS = 256;

template <int L>
__global__ __launch_bounds__(PREP_THREADS) void chunk_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k,
    const float* __restrict__ i_pre, const float* __restrict__ f_pre,
    int S, int dqk, Ws ws)
{
    constexpr int LB = L / 16;
    constexpr int PPITCH = L + 8;
    __shared__ double sb[L], sml[L];
    __shared__ float si[L];
    __shared__ double wsum[2], wmax[2];  // per-wave totals of the two scans (separate: no reuse race)
    __shared__ __attribute__((aligned(16))) bf16 sP[2][L * PPITCH];   // hi, lo

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lg = lane >> 4;
    const size_t tok0 = (size_t)bh * S + (size_t)c * L;

    // gates: cumulative log forget gate and chunk-local stabilizer, by wave scans (fp64)
    double lf = 0.0, ii = 0.0;
    if (tid < L) {
        lf = log_sigmoid_f64((double)f_pre[tok0 + tid]);
        ii = (double)i_pre[tok0 + tid];
    }
    double bcum = 0.0;
    if (wave < 2) {
        bcum = wave_scan_add(lf, lane);
        if (lane == 63) wsum[wave] = bcum;
    }
    __syncthreads();
    if (wave == 1) bcum += wsum[0];
    double umax = 0.0;
    if (wave < 2) {
        umax = wave_scan_max(tid < L ? ii - bcum : -INFINITY, lane);
        if (lane == 63) wmax[wave] = umax;
    }
    __syncthreads();
    if (wave == 1) umax = fmax(umax, wmax[0]);
    if (tid < L) {
        sb[tid] = bcum;
        si[tid] = (float)ii;
        sml[tid] = bcum + umax;
    }
    __syncthreads();
    if (tid < L) {
        const double bL = sb[L - 1], mL = sml[L - 1];
        ws.b[tok0 + tid] = sb[tid];
        ws.mloc[tok0 + tid] = sml[tid];
        ws.wloc[tok0 + tid] = exp_arg(bL - sb[tid] + (double)si[tid] - mL);
    }

    // decayed scores, one 16-row block per wave pass
    const bf16* qh = q + tok0 * dqk;
    const bf16* kh = k + tok0 * dqk;
    for (int tb = wave; tb < LB; tb += PREP_THREADS / 64) {
        const int rows_tb = tb;
        f32x4 den4 = {0, 0, 0, 0};
        for (int sbk = 0; sbk < LB; ++sbk) {
            f32x4 acc = {0, 0, 0, 0};
            if (sbk <= rows_tb) {
                const bf16* qa = qh + (size_t)(16 * rows_tb + ln) * dqk + 8 * lg;
                const bf16* kb = kh + (size_t)(16 * sbk + ln) * dqk + 8 * lg;
                for (int kk = 0; kk < dqk; kk += 32) {
                    bf16x8 a = *reinterpret_cast<const bf16x8*>(qa + kk);
                    bf16x8 bb = *reinterpret_cast<const bf16x8*>(kb + kk);
                    acc = mfma(a, bb, acc);
                }
            }
            const int s = 16 * sbk + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tau = 16 * rows_tb + 4 * lg + i;
                float p = 0.0f;
                if (s <= tau) p = acc[i] * exp_arg(sb[tau] - sb[s] + (double)si[s] - sml[tau]);
                den4[i] += p;
                const bf16 hi = (bf16)p;
                sP[0][tau * PPITCH + s] = hi;
                sP[1][tau * PPITCH + s] = (bf16)(p - (float)hi);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float d = den4[i];
            d += __shfl_xor(d, 1, 64);
            d += __shfl_xor(d, 2, 64);
            d += __shfl_xor(d, 4, 64);
            d += __shfl_xor(d, 8, 64);
            if (ln == 0) ws.den[tok0 + 16 * rows_tb + 4 * lg + i] = d;
        }
    }
    __syncthreads();
    // rows of P_loc (hi block, then lo block) out, 16 bytes per lane
    bf16* Pout = ws.P + 2 * tok0 * L;
    for (int idx = tid; idx < 2 * L * L / 8; idx += PREP_THREADS) {
        const int half = idx / (L * L / 8), rem = idx % (L * L / 8);
        const int row = rem / (L / 8), col = 8 * (rem % (L / 8));
        const bf16* src = sP[half] + row * PPITCH + col;
        bf16x8 v = bf16x8{src[0], src[1], src[2], src[3], src[4], src[5], src[6], src[7]};
        *reinterpret_cast<bf16x8*>(Pout + (size_t)half * L * L + (size_t)row * L + col) = v;
    }
}

// ---------------------------------------------------------------------------
// kernel 2: sequential scan over chunks, state in accumulators
// ---------------------------------------------------------------------------
// NC column blocks of 16 value columns x NK key parts = NC*NK waves per workgroup.
template <int L_, int DQ_, int NC_, int NK_, int SB_, int MINB_>
struct ScanCfg {
    static constexpr int L = L_, DQ = DQ_, NC = NC_, NK = NK_, SB = SB_;
    static constexpr int MINB = MINB_;     // workgroups per CU the register budget must allow
    static constexpr int W = NC * NK, THREADS = 64 * W, TV = 16 * NC;
    static constexpr int DP = DQ / NK;     // key rows owned by one wave
    static constexpr int NS = DP / SB;     // slabs per chunk
    static constexpr int SW = NK * SB;     // staged slab width (key columns)
    static constexpr int QP = SW + 4;      // Q pitch: row stride = 2 (mod 32) dwords
    static constexpr int KP = SW + 16;     // K pitch: row stride = 8 (mod 32) dwords
    static constexpr int VP = ((TV + 63) / 64) * 64 + 16;  // V pitch: 8 (mod 32) dwords
    static constexpr int LB = L / 16;      // 16-row blocks of a chunk
    static constexpr int SBB = SB / 16;    // state blocks per slab
    static constexpr int NSB = DP / 16;    // state blocks per wave
    static_assert(SW % 64 == 0, "slab width must be a multiple of 64 columns");
    static_assert(SB % 32 == 0 && DP % SB == 0, "slab must tile the key rows of a wave");
    static_assert(LB % NK == 0, "row blocks must split evenly over the key parts");
    static_assert(L % 32 == 0, "chunk must be a multiple of 32 tokens");
    static_assert(THREADS <= 1024, "workgroup too large");
};

template <class C>
struct alignas(16) ScanSmem {
    union alignas(16) {
        struct {
            alignas(16) bf16 q[C::L * C::QP];
            alignas(16) bf16 k[C::L * C::KP];
        } slab;
        float red[C::L * C::TV];     // Q C'^T summed over the key parts, in D layout
    } u;
    alignas(16) bf16 v[C::L * C::VP];     // V tile (for P V)
    alignas(16) bf16 vwh[C::L * C::VP];   // hi(w (.) V)
    alignas(16) bf16 vwl[C::L * C::VP];   // lo(w (.) V)
    float n[C::DQ];
    double b[C::L], mloc[C::L];          // fp64 gate arithmetic
    float denloc[C::L], wloc[C::L];
    float a[C::L], r[C::L], fl[C::L], w[C::L], den[C::L];
};

__device__ __forceinline__ void split8(f32x4 x0, f32x4 x1, bf16x8& hi, bf16x8& lo) {
    hi = cvt8(x0, x1);
    f32x4 r0 = x0 - f32x4{(float)hi[0], (float)hi[1], (float)hi[2], (float)hi[3]};
    f32x4 r1 = x1 - f32x4{(float)hi[4], (float)hi[5], (float)hi[6], (float)hi[7]};
    lo = cvt8(r0, r1);
}

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void chunk_scan_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ o_pre, Ws ws, int S, int dv, int n_vt, int remap,
    const float* __restrict__ C0, const float* __restrict__ n0, const float* __restrict__ m0,
    bf16* __restrict__ h, float* __restrict__ Cout, float* __restrict__ nout, float* __restrict__ mout)
{
    constexpr int L = C::L, DQ = C::DQ, NC = C::NC, NK = C::NK, SB = C::SB;
    constexpr int THREADS = C::THREADS, TV = C::TV, DP = C::DP, NS = C::NS, SW = C::SW;
    constexpr int QP = C::QP, KP = C::KP, VP = C::VP, LB = C::LB, SBB = C::SBB, NSB = C::NSB;
    __shared__ ScanSmem<C> sm;

    // workgroup -> (head, value tile); consecutive slots share an XCD when remapped
    int wg = blockIdx.x;
    if (remap) {
        const int G = gridDim.x;
        wg = (wg % 8) * (G / 8) + wg / 8;
    }
    const int bh = wg / n_vt, vt = wg % n_vt;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cb = wave % NC, kq = wave / NC;
    const int ln = lane & 15, lg = lane >> 4;
    const int vcol = vt * TV + 16 * cb;          // first value column of this wave
    const bool active = vcol < dv;
    const int vtile_cols = min(TV, dv - vt * TV); // valid columns of the tile

    const size_t tokh = (size_t)bh * S;
    const bf16* qh = q + tokh * DQ;
    const bf16* kh = k + tokh * DQ;
    const bf16* vh = v + tokh * dv;
    const float* oh = o_pre + tokh * dv;
    bf16* hh = h + tokh * dv;

    // state: block jb holds key rows j = kq*DP + 16*jb + 4*lg + i, value column vcol + ln
    f32x4 st[NSB];
#pragma unroll
    for (int jb = 0; jb < NSB; ++jb) {
        st[jb] = f32x4{0, 0, 0, 0};
        if (C0 && active)
            st[jb] = *reinterpret_cast<const f32x4*>(
                C0 + ((size_t)bh * dv + vcol + ln) * DQ + kq * DP + 16 * jb + 4 * lg);
    }
    for (int j = tid; j < DQ; j += THREADS) sm.n[j] = n0 ? n0[(size_t)bh * DQ + j] : 0.0f;
    double m_prev = m0 ? (double)m0[bh] : 0.0;

    const int n_chunks = S / L;
    for (int c = 0; c < n_chunks; ++c) {
        const size_t t0 = (size_t)c * L;
        // --- stage gates and the V tile -----------------------------------
        for (int i = tid; i < L; i += THREADS) {
            sm.b[i] = ws.b[tokh + t0 + i];
            sm.mloc[i] = ws.mloc[tokh + t0 + i];
            sm.denloc[i] = ws.den[tokh + t0 + i];
            sm.wloc[i] = ws.wloc[tokh + t0 + i];
        }
        for (int idx = tid; idx < L * TV / 8; idx += THREADS) {
            const int row = idx / (TV / 8), col = 8 * (idx % (TV / 8));
            bf16x8 x = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (col < vtile_cols)
                x = *reinterpret_cast<const bf16x8*>(vh + (t0 + row) * dv + vt * TV + col);
            *reinterpret_cast<bf16x8*>(sm.v + row * VP + col) = x;
        }
        __syncthreads();
        // --- per-token stabilizer terms -------------------------------------
        const double bL = sm.b[L - 1], mlocL = sm.mloc[L - 1];
        const double mL = fmax(bL + m_prev, mlocL);
        const float alpha = exp_arg(bL + m_prev - mL);
        const float rL = exp_arg(mlocL - mL);
        for (int i = tid; i < L; i += THREADS) {
            const double mt = fmax(sm.b[i] + m_prev, sm.mloc[i]);
            sm.fl[i] = exp_arg(-mt);                  // floor of |den|: exp(-m_t)
            sm.a[i] = exp_arg(sm.b[i] + m_prev - mt);
            sm.r[i] = exp_arg(sm.mloc[i] - mt);
            sm.w[i] = rL * sm.wloc[i];
            sm.den[i] = 0.0f;
        }
        __syncthreads();
        // w (.) V split into bf16 hi + lo
        for (int idx = tid; idx < L * TV / 8; idx += THREADS) {
            const int row = idx / (TV / 8), col = 8 * (idx % (TV / 8));
            const float ws_ = sm.w[row];
            const bf16* src = sm.v + row * VP + col;
            bf16x8 xh, xl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = ws_ * (float)src[e];
                xh[e] = (bf16)x;
                xl[e] = (bf16)(x - (float)xh[e]);
            }
            *reinterpret_cast<bf16x8*>(sm.vwh + row * VP + col) = xh;
            *reinterpret_cast<bf16x8*>(sm.vwl + row * VP + col) = xl;
        }
        // (the first slab barrier below also publishes vwh / vwl)

        f32x4 acc_inter[LB];
#pragma unroll
        for (int tb = 0; tb < LB; ++tb) acc_inter[tb] = f32x4{0, 0, 0, 0};

#pragma unroll
        for (int s = 0; s < NS; ++s) {
            // --- stage Q and K slab s (NK pieces of SB key columns) ----------
            for (int idx = tid; idx < L * SW / 8; idx += THREADS) {
                const int row = idx / (SW / 8), c8 = 8 * (idx % (SW / 8));
                const int part = c8 / SB, jcol = part * DP + s * SB + (c8 % SB);
                bf16x8 xq = *reinterpret_cast<const bf16x8*>(qh + (t0 + row) * DQ + jcol);
                bf16x8 xk = *reinterpret_cast<const bf16x8*>(kh + (t0 + row) * DQ + jcol);
                bf16* dq = sm.u.slab.q + row * QP + c8;   // 8-byte aligned rows
                *reinterpret_cast<bf16x4*>(dq) = bf16x4{xq[0], xq[1], xq[2], xq[3]};
                *reinterpret_cast<bf16x4*>(dq + 4) = bf16x4{xq[4], xq[5], xq[6], xq[7]};
                *reinterpret_cast<bf16x8*>(sm.u.slab.k + row * KP + c8) = xk;
            }
            __syncthreads();
            if (active) {
                // inter-chunk retrieval: acc_inter += Q[:, slab] (C'_hi + C'_lo)^T[slab, cols]
#pragma unroll
                for (int kk = 0; kk < SB / 32; ++kk) {
                    bf16x8 bhi, blo;
                    split8(st[s * SBB + 2 * kk], st[s * SBB + 2 * kk + 1], bhi, blo);
#pragma unroll
                    for (int tb = 0; tb < LB; ++tb) {
                        const bf16* qa = sm.u.slab.q + (16 * tb + ln) * QP + kq * SB + 32 * kk + 4 * lg;
                        const bf16x8 aop = cat(*reinterpret_cast<const bf16x4*>(qa),
                                               *reinterpret_cast<const bf16x4*>(qa + 16));
                        acc_inter[tb] = mfma(aop, bhi, acc_inter[tb]);
                        acc_inter[tb] = mfma(aop, blo, acc_inter[tb]);
                    }
                }
                // state update: C'^T[slab] = alpha C'^T[slab] + K[:, slab]^T (w V)_{hi+lo}
#pragma unroll
                for (int jb = 0; jb < SBB; ++jb) st[s * SBB + jb] *= alpha;
#pragma unroll
                for (int kk = 0; kk < L / 32; ++kk) {
                    // B operands: rows (tokens) 32kk + 8lg + 0..7 of w V, column vcol + ln
                    const int vrow = (32 * kk + 8 * lg + (ln >> 2)) * VP + 16 * cb + 4 * (ln & 3);
                    const bf16x8 bhi = cat(lds_read_tr(sm.vwh + vrow), lds_read_tr(sm.vwh + vrow + 4 * VP));
                    const bf16x8 blo = cat(lds_read_tr(sm.vwl + vrow), lds_read_tr(sm.vwl + vrow + 4 * VP));
#pragma unroll
                    for (int jb = 0; jb < SBB; ++jb) {
                        const bf16* ka = sm.u.slab.k + (32 * kk + 8 * lg + (ln >> 2)) * KP + kq * SB + 16 * jb + 4 * (ln & 3);
                        const bf16x8 aop = cat(lds_read_tr(ka), lds_read_tr(ka + 4 * KP));
                        st[s * SBB + jb] = mfma(aop, bhi, st[s * SBB + jb]);
                        st[s * SBB + jb] = mfma(aop, blo, st[s * SBB + jb]);
                    }
                }
            }
            // normalizer, inter part: den[tau] += Q[tau, slab] . n'[slab]  (16 lanes per row)
            for (int idx = tid; idx < L * 16; idx += THREADS) {
                const int tau = idx >> 4, lp = idx & 15;
                constexpr int CPL = SW / 16;  // columns per lane
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int cc = lp * CPL + e;
                    const int j = (cc / SB) * DP + s * SB + (cc % SB);
                    acc += (float)sm.u.slab.q[tau * QP + cc] * sm.n[j];
                }
                acc += __shfl_xor(acc, 1, 64);
                acc += __shfl_xor(acc, 2, 64);
                acc += __shfl_xor(acc, 4, 64);
                acc += __shfl_xor(acc, 8, 64);
                if (lp == 0) sm.den[tau] += acc;
            }
            __syncthreads();
            // normalizer state: n'[slab] = alpha n' + K[:, slab]^T w
            for (int cc = tid; cc < SW; cc += THREADS) {
                const int j = (cc / SB) * DP + s * SB + (cc % SB);
                float acc = 0.0f;
                for (int t = 0; t < L; ++t) acc += sm.w[t] * (float)sm.u.slab.k[t * KP + cc];
                sm.n[j] = alpha * sm.n[j] + acc;
            }
            __syncthreads();
        }

        // --- sum Q C'^T over the key parts in a fixed order (deterministic) ----
        if (NK > 1) {
#pragma unroll
            for (int kp = 0; kp < NK; ++kp) {
                if (kq == kp && active) {
#pragma unroll
                    for (int tb = 0; tb < LB; ++tb) {
                        f32x4* dst = reinterpret_cast<f32x4*>(sm.u.red + (tb * NC + cb) * 256 + lane * 4);
                        *dst = (kp == 0) ? acc_inter[tb] : (*dst + acc_inter[tb]);
                    }
                }
                __syncthreads();
            }
        }
        // --- intra-chunk product, normalize, gate, store (part kq owns tb % NK == kq) ---
        if (active) {
            const bf16* Pc = ws.P + 2 * (tokh + t0) * L;   // hi block, then lo block
#pragma unroll
            for (int tb = 0; tb < LB; ++tb) {
                if (tb % NK != kq) continue;
                const f32x4 inter = (NK > 1)
                    ? *reinterpret_cast<const f32x4*>(sm.u.red + (tb * NC + cb) * 256 + lane * 4)
                    : acc_inter[tb];
                // intra: (P_hi + P_lo)[rows of tb, s <= last row of tb] V[:, cols]
                f32x4 intra = {0, 0, 0, 0};
                for (int kk = 0; kk <= (16 * tb + 15) / 32; ++kk) {
                    const bf16* pa = Pc + (size_t)(16 * tb + ln) * L + 32 * kk + 8 * lg;
                    const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(pa);
                    const bf16x8 alo = *reinterpret_cast<const bf16x8*>(pa + L * L);
                    const bf16* vb = sm.v + (32 * kk + 8 * lg + (ln >> 2)) * VP + 16 * cb + 4 * (ln & 3);
                    const bf16x8 bop = cat(lds_read_tr(vb), lds_read_tr(vb + 4 * VP));
                    intra = mfma(ahi, bop, intra);
                    intra = mfma(alo, bop, intra);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tau = 16 * tb + 4 * lg + i;
                    const float ra = sm.r[tau], aa = sm.a[tau];
                    const float num = ra * intra[i] + aa * inter[i];
                    const float den = ra * sm.denloc[tau] + aa * sm.den[tau];
                    const size_t o = (t0 + tau) * dv + vcol + ln;
                    const float hv = sigmoid(oh[o]) * num / fmaxf(fabsf(den), sm.fl[tau]);
                    hh[o] = (bf16)hv;
                }
            }
        }
        m_prev = mL;
        __syncthreads();
    }

    // final stabilized state
    if (active) {
#pragma unroll
        for (int jb = 0; jb < NSB; ++jb)
            *reinterpret_cast<f32x4*>(Cout + ((size_t)bh * dv + vcol + ln) * DQ + kq * DP + 16 * jb + 4 * lg) = st[jb];
    }
    if (vt == 0) {
        for (int j = tid; j < DQ; j += THREADS) nout[(size_t)bh * DQ + j] = sm.n[j];
        if (tid == 0) mout[bh] = (float)m_prev;
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int L>
hipError_t launch_prep(const FwdArgs& a, const Ws& w) {
    dim3 grid(a.S / L, a.B * a.NH);
    hipLaunchKernelGGL((chunk_prep_kernel<L>), grid, dim3(PREP_THREADS), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, a.i_pre, a.f_pre, a.S, a.dqk, w);
    return hipGetLastError();
}

template <class C>
hipError_t launch_scan(const FwdArgs& a, const Ws& w) {
    const int n_vt = (a.dv + C::TV - 1) / C::TV;
    const int G = a.B * a.NH * n_vt;
    const int remap = (G % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_scan_kernel<C>), dim3(G), dim3(C::THREADS), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.o_pre, w, a.S, a.dv, n_vt, remap,
                       a.C0, a.n0, a.m0, (bf16*)a.h, a.C, a.n, a.m);
    return hipGetLastError();
}

template <int L, int DQ, int NC, int NK, int SB, int MINB>
hipError_t run(const FwdArgs& a) {
    Ws w = ws_layout(a.ws, (size_t)a.B * a.NH, a.S, L);
    hipError_t e = launch_prep<L>(a, w);
    if (e != hipSuccess) return e;
    return launch_scan<ScanCfg<L, DQ, NC, NK, SB, MINB>>(a, w);
}

typedef hipError_t (*RunFn)(const FwdArgs&);

// supported (chunk, d_qk) pairs and the tiling used for each
RunFn pick(int L, int dqk) {
#define MLSTM_CASE(L_, DQ_, NC_, NK_, SB_, MINB_) \
    if (L == L_ && dqk == DQ_) return &run<L_, DQ_, NC_, NK_, SB_, MINB_>;
    // (chunk, d_qk, column blocks, key parts, slab, workgroups per CU)
    MLSTM_CASE(32, 128, 4, 1, 128, 1)
    MLSTM_CASE(32, 384, 3, 2, 64, 1)
    MLSTM_CASE(64, 128, 4, 1, 128, 1)
    MLSTM_CASE(64, 256, 4, 2, 64, 1)
    MLSTM_CASE(64, 384, 3, 4, 32, 1)
    MLSTM_CASE(64, 512, 4, 2, 64, 1)
    MLSTM_CASE(64, 1024, 2, 2, 64, 2)
    MLSTM_CASE(128, 128, 4, 2, 32, 1)
    MLSTM_CASE(128, 256, 4, 2, 32, 1)
#undef MLSTM_CASE
    return nullptr;
}

}  // namespace

bool mfma_fwd_supported(const FwdArgs& a) {
    return a.dtype == MLSTM_BF16 && a.S % a.chunk == 0 && pick(a.chunk, a.dqk) != nullptr;
}

size_t mfma_fwd_workspace_bytes(const FwdArgs& a) {
    return ws_bytes((size_t)a.B * a.NH, a.S, a.chunk);
}

hipError_t launch_fwd_mfma(const FwdArgs& a) {
    RunFn f = pick(a.chunk, a.dqk);
    if (!f) return hipErrorNotSupported;
    return f(a);
}

}  // namespace mlstm
