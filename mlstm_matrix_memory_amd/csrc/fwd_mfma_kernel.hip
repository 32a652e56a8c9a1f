// Chunkwise parallel forward of the mLSTM cell on bf16 MFMA (gfx950).
//
// "xLSTM: Extended Long Short-Term Memory": section 2.3 (covariance update
// eq. (18), normalizer with floor, multi-head independence and the parallel form
// of the recurrence) and section 2.2 (stabilizer m_t, eq. (17)).
//
// Two stages.  The prepare stage is parallel over chunks: chunk_prep (below),
// then gate_scan (the stabilizer and normalizer carried across chunks, which fix
// every per-token weight) and den_kernel (the full normalizer n'.q of every row).
// The scan stage is sequential over chunks: chunk_scan2 (pipelined form), or at
// d_qk 512 and 1024 chunk_scan4 (streaming form, see its comment), preceded for
// few heads over long sequences by seg_state and seg_combine, which let
// independent sequence segments start from their own entering states.  The two
// kernels that carry the work, both on bf16 MFMA with fp32 accumulation:
//
// 1. chunk_prep (one workgroup per (head, chunk), all chunks in parallel)
//      b_tau     = in-chunk cumulative sum of log sigmoid(f~)
//      m_loc_tau = b_tau + max_{s<=tau}(i~_s - b_s)          chunk-local row max
//      P_loc     = (Q K^T) (.) exp(b_tau - b_s + i~_s - m_loc_tau)   (s <= tau)
//      den_loc   = rowsum(P_loc) (fp32),  w_loc_s = exp(b_L - b_s + i~_s - m_loc_L)
//    P_loc is stored in bf16 (it is the MFMA operand of the next kernel); every
//    exponent is <= 0 so nothing overflows.
//
// 2. chunk_scan2 (one workgroup per (head, segment, tile of TV value columns),
//    sequential over the chunks of the segment, state carried in MFMA accumulators)
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
#include <climits>
#include <type_traits>

namespace mlstm {
namespace {


__device__ __forceinline__ bf16x8 cvt8(f32x4 a, f32x4 b) {
    return bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3],
                  (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
}

// Two floats to a pair of bf16 (round to nearest even), first in the low half.
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
__device__ __forceinline__ unsigned pk2(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// x = hi + lo for eight floats.  Each pair is rounded once into its packed hi word
// and the two hi values are read back from that word's halves (a shift and a mask),
// so a float costs one subtraction and two half-conversions besides.
__device__ __forceinline__ void split8(f32x4 x0, f32x4 x1, bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float a = i < 2 ? x0[2 * i] : x1[2 * i - 4], b = i < 2 ? x0[2 * i + 1] : x1[2 * i - 3];
        h[i] = pk2(a, b);
        l[i] = pk2(a - __builtin_bit_cast(float, h[i] << 16), b - __builtin_bit_cast(float, h[i] & 0xffff0000u));
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// x = hi + lo for the products w * v of one weight and eight bf16 values
__device__ __forceinline__ void split8w(float w, bf16x8 v, bf16x8& hi, bf16x8& lo) {
    split8(f32x4{w * (float)v[0], w * (float)v[1], w * (float)v[2], w * (float)v[3]},
           f32x4{w * (float)v[4], w * (float)v[5], w * (float)v[6], w * (float)v[7]}, hi, lo);
}

// Sum over the 16 lanes of each row of a wave with DPP lane permutes (VALU only,
// no LDS round trips): swap neighbours, swap pairs, mirror within 8, mirror within 16.
__device__ __forceinline__ float row16_sum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false)); // row_half_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false)); // row_mirror
    return x;
}

// Lane (quad lane b = lane & 3) reads x from quad lane (b + R) & 3 (DPP quad_perm).
template <int R>
__device__ __forceinline__ float quad_rotate(float x) {
    constexpr int ctrl = ((0 + R) & 3) | (((1 + R) & 3) << 2) | (((2 + R) & 3) << 4) | (((3 + R) & 3) << 6);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), ctrl, 0xF, 0xF, false));
}

// 4 x 4 transpose within each quad of lanes.  In the MFMA accumulator layout, quad
// lane b holds rows 4g..4g+3 (g = lane / 16) of column 4a + b (a = (lane % 16) / 4);
// afterwards it holds row 4g + b at columns 4a..4a+3, so one 8-byte store writes it.
// Two exchange stages: lanes b and b ^ 2 swap the registers whose index differs from
// b in bit 1, then lanes b and b ^ 1 those that differ in bit 0 (a swap of two
// registers each way per stage: two DPP moves and six selects).
__device__ __forceinline__ f32x4 quad_transpose(f32x4 y, int b) {
    const bool b2 = (b & 2) != 0, b1 = (b & 1) != 0;
    const float s0 = b2 ? y[0] : y[2], s1 = b2 ? y[1] : y[3];
    const float r0 = quad_rotate<2>(s0), r1 = quad_rotate<2>(s1);     // from lane b ^ 2
    const f32x4 z = {b2 ? r0 : y[0], b2 ? r1 : y[1], b2 ? y[2] : r0, b2 ? y[3] : r1};
    const float u0 = b1 ? z[0] : z[1], u1 = b1 ? z[2] : z[3];
    const float q0 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, u0), 0xB1, 0xF, 0xF, false));
    const float q1 = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, u1), 0xB1, 0xF, 0xF, false));
    return f32x4{b1 ? q0 : z[0], b1 ? z[1] : q0, b1 ? q1 : z[2], b1 ? z[3] : q1};   // from lane b ^ 1
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
// workspace layout (one allocation, 256-byte aligned pieces)
// ---------------------------------------------------------------------------
struct Ws {
    bf16* P;        // [heads][chunk][2][L][L]  decayed intra-chunk scores, bf16 hi then lo
    double* b;      // [heads][S]  in-chunk cumulative log forget gate
    double* mloc;   // [heads][S]  chunk-local stabilizer
    float* den;     // [heads][S]  row sums of the decayed scores (fp32, before rounding)
    float* wloc;    // [heads][S]  chunk-local update weights
    float* dn;      // [heads][chunk][DQ]  K^T w_loc of each chunk
    // six per-token arrays in one allocation [6][heads][S], in this order (the scan
    // stages the first three with every chunk):
    float* a;       // weight of the carried state in each row
    float* r;       // rescale of the chunk-local scores to the carried stabilizer
    float* rden;    // 1 / max(|n'.q|, exp(-m_t)): the divisor of each row, inverted
    float* fl;      // floor exp(-m_t) of the normalizer
    float* w;       // update weights with the carried stabilizer
    float* alt;     // alpha of the token's chunk, repeated over its tokens
    size_t hs;      // heads * S: stride between the six arrays
    float* alpha;   // [heads][chunk]  decay of the carried state across the chunk
    float* nent;    // [heads][chunk][DQ]  normalizer n' entering each chunk
    float* nfin;    // [heads][DQ]  final normalizer
    float* mfin;    // [heads]      final stabilizer
    float* cst;     // [heads][G][DV][DQ]  state entering each sequence segment (slot 0: the initial one)
    float* cpart;   // [heads][G-1][SP][DV][DQ]  sums over the SP token parts of each segment but the last
    int sp;         // token parts per segment in seg_state_kernel
    // Q and K of each 64-token chunk in MFMA operand order (streaming scan only, else
    // null): [heads][chunk][DQ/32][4][64 lanes][8], one 1 KB fragment per 32-key step
    // and operand block, so that a wave reads each fragment as one contiguous load
    bf16* qs;
    bf16* ks;
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Token parts per segment for the segment sums: enough workgroups for two per CU,
// each part at least 4 chunks long.
constexpr int SS_TILE = 128;           // key rows and value columns of a segment-sum workgroup's tile
constexpr int SS_MAXP = 8;
inline int seg_parts(size_t heads, size_t nC, int DQ, int DV, int G) {
    if (G <= 1) return 1;
    const size_t tiles = (size_t)((DQ + SS_TILE - 1) / SS_TILE) * ((DV + SS_TILE - 1) / SS_TILE);
    const size_t nCs = nC / G;
    int P = 1;
    while (2 * P <= SS_MAXP && tiles * (G - 1) * heads * P < 512 && nCs % (2 * P) == 0 && nCs / (2 * P) >= 4) P *= 2;
    return P;
}

inline size_t ws_walk(void* base, size_t heads, size_t S, int L, int DQ, int DV, int G, bool kt, Ws* out) {
    const size_t nC = S / L;
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t bytes) { char* q = p + off; off += align256(bytes); return q; };
    Ws w;
    w.P = (bf16*)take(2 * heads * S * L * sizeof(bf16));
    w.b = (double*)take(heads * S * sizeof(double));
    w.mloc = (double*)take(heads * S * sizeof(double));
    w.den = (float*)take(heads * S * sizeof(float));
    w.wloc = (float*)take(heads * S * sizeof(float));
    w.dn = (float*)take(heads * nC * DQ * sizeof(float));
    w.hs = heads * S;
    w.a = (float*)take(6 * heads * S * sizeof(float));
    w.r = w.a + w.hs;
    w.rden = w.a + 2 * w.hs;
    w.fl = w.a + 3 * w.hs;
    w.w = w.a + 4 * w.hs;
    w.alt = w.a + 5 * w.hs;
    w.alpha = (float*)take(heads * nC * sizeof(float));
    w.nent = (float*)take(heads * nC * DQ * sizeof(float));
    w.nfin = (float*)take(heads * DQ * sizeof(float));
    w.mfin = (float*)take(heads * sizeof(float));
    w.cst = G > 1 ? (float*)take(heads * G * (size_t)DV * DQ * sizeof(float)) : nullptr;
    w.sp = seg_parts(heads, nC, DQ, DV, G);
    w.cpart = G > 1 ? (float*)take(heads * (G - 1) * (size_t)w.sp * DV * DQ * sizeof(float)) : nullptr;
    w.qs = kt ? (bf16*)take(heads * S * DQ * sizeof(bf16)) : nullptr;
    w.ks = kt ? (bf16*)take(heads * S * DQ * sizeof(bf16)) : nullptr;
    if (out) *out = w;
    return off;
}
inline Ws ws_layout(void* base, size_t heads, size_t S, int L, int DQ, int DV, int G, bool kt) {
    Ws w;
    ws_walk(base, heads, S, L, DQ, DV, G, kt, &w);
    return w;
}
inline size_t ws_bytes(size_t heads, size_t S, int L, int DQ, int DV, int G, bool kt) {
    return ws_walk(nullptr, heads, S, L, DQ, DV, G, kt, nullptr);
}

// ---------------------------------------------------------------------------
// kernel 1: per-chunk gates and intra-chunk decayed scores
// ---------------------------------------------------------------------------
constexpr int PREP_THREADS = 256;
constexpr int PREP_SB = 64;                 // key columns per staged slab of Q and K
constexpr int PREP_KP = PREP_SB + 8;        // LDS row pitch (bf16): 36 dwords, b128 operand reads conflict free

template <int L>
struct alignas(16) PrepSmem {
    alignas(16) bf16 q[L * PREP_KP];
    alignas(16) bf16 k[L * PREP_KP];
    double sb[L], sml[L];
    float si[L], swl[L];
    float red[4][PREP_SB];
    double wsum[2], wmax[2];  // per-wave totals of the two scans (separate: no reuse race)
};

// Q and K of the chunk are staged through LDS one slab of key columns at a time
// (each element is read from HBM once); the next slab is already in flight in
// registers while the current one is multiplied.  Wave w owns the 16-row blocks
// tb = w, w + 4, ... of the score matrix with all their causal column blocks, so
// every row sum is formed inside one wave in a fixed order.
template <int L, bool FRAG>
__global__ __launch_bounds__(PREP_THREADS) void chunk_prep_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k,
    const float* __restrict__ i_pre, const float* __restrict__ f_pre,
    int S, int Sx, int dqk, Ws ws)
{
    constexpr int LB = L / 16;
    constexpr int NW = PREP_THREADS / 64;
    constexpr int TBW = (LB + NW - 1) / NW;          // row blocks per wave
    constexpr int UNITS = L * PREP_SB / 8;           // 16-byte units of one slab of Q (or K)
    constexpr int UPT = (2 * UNITS + PREP_THREADS - 1) / PREP_THREADS;
    __shared__ PrepSmem<L> sm;

    const int c = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int ln = lane & 15, lg = lane >> 4;
    const size_t tok0 = (size_t)bh * S + (size_t)c * L;     // workspace token index
    const size_t tin0 = (size_t)bh * Sx + (size_t)c * L;    // input token index
    const bf16* qh = q + tin0 * dqk;
    const bf16* kh = k + tin0 * dqk;

    auto slab_load = [&](f32x4 (&reg)[UPT], int j0) {
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = tid + u * PREP_THREADS;
            if (idx < 2 * UNITS) {
                const int which = idx / UNITS, rem = idx % UNITS;
                const int row = rem / (PREP_SB / 8), c8 = 8 * (rem % (PREP_SB / 8));
                reg[u] = *reinterpret_cast<const f32x4*>((which ? kh : qh) + (size_t)row * dqk + j0 + c8);
            }
        }
    };
    f32x4 reg[UPT];
    slab_load(reg, 0);

    // gates: cumulative log forget gate and chunk-local stabilizer, by wave scans (fp64)
    double lf = 0.0, ii = 0.0;
    if (tid < L) {
        lf = log_sigmoid_f64((double)f_pre[tin0 + tid]);
        ii = (double)i_pre[tin0 + tid];
    }
    double bcum = 0.0;
    if (wave < 2) {
        bcum = wave_scan_add(lf, lane);
        if (lane == 63) sm.wsum[wave] = bcum;
    }
    __syncthreads();
    if (wave == 1) bcum += sm.wsum[0];
    double umax = 0.0;
    if (wave < 2) {
        umax = wave_scan_max(tid < L ? ii - bcum : -INFINITY, lane);
        if (lane == 63) sm.wmax[wave] = umax;
    }
    __syncthreads();
    if (wave == 1) umax = fmax(umax, sm.wmax[0]);
    if (tid < L) {
        sm.sb[tid] = bcum;
        sm.si[tid] = (float)ii;
        sm.sml[tid] = bcum + umax;
    }
    __syncthreads();
    if (tid < L) {
        const double bL = sm.sb[L - 1], mL = sm.sml[L - 1];
        ws.b[tok0 + tid] = sm.sb[tid];
        ws.mloc[tok0 + tid] = sm.sml[tid];
        const float wl = exp_arg(bL - sm.sb[tid] + (double)sm.si[tid] - mL);
        ws.wloc[tok0 + tid] = wl;
        sm.swl[tid] = wl;
    }

    f32x4 acc[TBW][LB];
#pragma unroll
    for (int r = 0; r < TBW; ++r)
#pragma unroll
        for (int sbk = 0; sbk < LB; ++sbk) acc[r][sbk] = f32x4{0, 0, 0, 0};
    float* dn = ws.dn + ((size_t)bh * (S / L) + c) * dqk;

    for (int j0 = 0; j0 < dqk; j0 += PREP_SB) {
        __syncthreads();   // previous slab fully consumed
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = tid + u * PREP_THREADS;
            if (idx < 2 * UNITS) {
                const int which = idx / UNITS, rem = idx % UNITS;
                const int row = rem / (PREP_SB / 8), c8 = 8 * (rem % (PREP_SB / 8));
                *reinterpret_cast<f32x4*>((which ? sm.k : sm.q) + row * PREP_KP + c8) = reg[u];
            }
        }
        __syncthreads();
        if (j0 + PREP_SB < dqk) slab_load(reg, j0 + PREP_SB);
        if constexpr (FRAG) {
            // the slab's fragments in MFMA operand order (64-token chunks): per 32-key
            // step ks, Q block tb (lane (ln, lg): row 16 tb + ln, keys 8 lg .. + 7) and
            // K^T block (jt, kk) (lane: key 8 (ln / 4) + 4 jt + ln % 4, tokens
            // 32 kk + 8 lg .. + 7, from two transposing reads)
            const size_t fr0 = (tok0 * dqk + (size_t)j0 * L) * 2;        // bytes
#pragma unroll
            for (int pr = wave; pr < 2 * (PREP_SB / 32) * 4; pr += NW) {
                const int isk = pr / ((PREP_SB / 32) * 4), rem = pr % ((PREP_SB / 32) * 4);
                const int kst = rem / 4, f = rem % 4;
                bf16x8 frag;
                if (!isk) {
                    frag = *reinterpret_cast<const bf16x8*>(sm.q + (16 * f + ln) * PREP_KP + 32 * kst + 8 * lg);
                } else {
                    const int jt = f / 2, kk = f % 2;
                    const bf16* kp = sm.k + (32 * kk + 8 * lg + (ln >> 2)) * PREP_KP + 32 * kst + 8 * (ln & 3) + 4 * jt;
                    frag = cat(lds_read_tr(kp), lds_read_tr(kp + 4 * PREP_KP));
                }
                char* dst = reinterpret_cast<char*>(isk ? ws.ks : ws.qs) + fr0 + ((size_t)kst * 4 + f) * 1024 + lane * 16;
                *reinterpret_cast<bf16x8*>(dst) = frag;
            }
        }
        // raw scores of this wave's causal blocks, contracted over the slab
#pragma unroll
        for (int r = 0; r < TBW; ++r) {
            const int tb = wave + NW * r;
            if (tb >= LB) continue;
#pragma unroll
            for (int kk = 0; kk < PREP_SB / 32; ++kk) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(sm.q + (16 * tb + ln) * PREP_KP + 32 * kk + 8 * lg);
#pragma unroll
                for (int sbk = 0; sbk < LB; ++sbk) {
                    if (sbk > tb) continue;
                    const bf16x8 bb = *reinterpret_cast<const bf16x8*>(sm.k + (16 * sbk + ln) * PREP_KP + 32 * kk + 8 * lg);
                    acc[r][sbk] = mfma(a, bb, acc[r][sbk]);
                }
            }
        }
        // chunk contribution to the normalizer, K^T w_loc, for this slab's columns (fp32)
        {
            const int col = tid % PREP_SB, part = tid / PREP_SB;
            constexpr int RP = L / (PREP_THREADS / PREP_SB);
            float acc_n = 0.0f;
#pragma unroll 8
            for (int t = part * RP; t < (part + 1) * RP; ++t) acc_n += sm.swl[t] * (float)sm.k[t * PREP_KP + col];
            sm.red[part][col] = acc_n;
        }
        __syncthreads();
        if (tid < PREP_SB) {
            float v = 0.0f;
#pragma unroll
            for (int part = 0; part < PREP_THREADS / PREP_SB; ++part) v += sm.red[part][tid];
            dn[j0 + tid] = v;
        }
    }

    // decay, row sums (fp32, before rounding), and P_loc out as bf16 hi then lo:
    // row-major, or for the streaming scan in MFMA operand order, staged through the
    // (now free) Q and K tiles
    constexpr bool frag = FRAG;
    bf16* Pout = ws.P + 2 * tok0 * L;
#pragma unroll
    for (int r = 0; r < TBW; ++r) {
        const int tb = wave + NW * r;
        if (tb >= LB) continue;
        f32x4 den4 = {0, 0, 0, 0};
#pragma unroll
        for (int sbk = 0; sbk < LB; ++sbk) {
            const int s = 16 * sbk + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tau = 16 * tb + 4 * lg + i;
                float p = 0.0f;
                if (sbk <= tb && s <= tau)
                    p = acc[r][sbk][i] * exp_arg(sm.sb[tau] - sm.sb[s] + (double)sm.si[s] - sm.sml[tau]);
                den4[i] += p;
                const bf16 hi = (bf16)p, lo = (bf16)(p - (float)hi);
                if constexpr (frag) {
                    sm.q[tau * PREP_KP + s] = hi;
                    sm.k[tau * PREP_KP + s] = lo;
                } else {
                    Pout[(size_t)tau * L + s] = hi;
                    Pout[(size_t)L * L + (size_t)tau * L + s] = lo;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = row16_sum(den4[i]);
            if (ln == 0) ws.den[tok0 + 16 * tb + 4 * lg + i] = d;
        }
    }
    if constexpr (frag) {
        // fragment (tb, kk, hl) at ((tb * 2 + kk) * 2 + hl) KB of the chunk's 16 KB:
        // lane (ln, lg) holds row 16 tb + ln, columns 32 kk + 8 lg .. + 7
        __syncthreads();
#pragma unroll
        for (int f = wave; f < 16; f += NW) {
            const int tb = f / 4, kk = (f / 2) % 2, hl = f % 2;
            const bf16* src = (hl ? sm.k : sm.q) + (16 * tb + ln) * PREP_KP + 32 * kk + 8 * lg;
            *reinterpret_cast<bf16x8*>(reinterpret_cast<char*>(Pout) + f * 1024 + lane * 16) =
                *reinterpret_cast<const bf16x8*>(src);
        }
    }
}

// ---------------------------------------------------------------------------
// kernel 1b: per head, the stabilizer and normalizer carried across chunks
// ---------------------------------------------------------------------------
// m entering chunk c follows the max-plus recurrence m <- max(b_L + m, m_loc_L);
// with it every per-token weight of the scan is fixed:
//   a_t = exp(b_t + m_p - m_t), r_t = exp(m_loc_t - m_t), fl_t = exp(-m_t),
//   w_t = exp(m_loc_L - m_L) w_loc_t, alpha_c = exp(b_L + m_p - m_L),
// and the normalizer entering each chunk follows n' <- alpha n' + exp(m_loc_L - m_L) K^T w_loc.
constexpr int GS_WAVES = 8;
constexpr int GS_THREADS = 64 * GS_WAVES;
constexpr int GS_COLS = 64;      // key columns of the normalizer per workgroup (one per lane)
constexpr int GS_TILE = 512;     // chunks per pass over LDS
constexpr int GS_BATCH = 16;     // loads issued together before their results are used

// The stabilizer recurrence m <- max(b_L + m, m_loc_L) is a max-plus affine map
// m -> max(A + m, B); maps compose as (A1, B1) then (A2, B2) = (A1 + A2, max(B1 + A2, B2)),
// so one wave scans a tile of chunks in parallel (each lane first composes a run
// of consecutive chunks, then the lanes combine by an inclusive shuffle scan).
// The normalizer recurrence n' <- alpha n' + rl dn is affine too: each wave
// carries it over its own range of chunks from zero, the ranges are chained
// through LDS, and each wave then walks its range again from the true value.
// Grid (parts, heads): every workgroup of a head repeats the short stabilizer
// scan and writes the per-token weights of its share of the tokens; the first
// d_qk/64 parts also carry the normalizer for their 64 key columns.  There are at
// least enough parts for one workgroup per CU (few heads over long sequences would
// otherwise leave the per-token work to a handful of workgroups).
template <int L>
__global__ __launch_bounds__(GS_THREADS) void gate_scan_kernel(Ws ws, int S, int dqk,
                                                               const float* __restrict__ n0,
                                                               const float* __restrict__ m0)
{
    __shared__ double sbl[GS_TILE], sml[GS_TILE], smp[GS_TILE + 1];
    __shared__ float salpha[GS_TILE], srl[GS_TILE];
    __shared__ float spart[GS_WAVES][GS_COLS], sprod[GS_WAVES], sfin[GS_COLS];
    const int part = blockIdx.x, nparts = gridDim.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int nC = S / L;
    const size_t tokh = (size_t)bh * S;
    const int j = part * GS_COLS + lane;
    double m_run = m0 ? (double)m0[bh] : 0.0;
    float n_in = (j < dqk && n0) ? n0[(size_t)bh * dqk + j] : 0.0f;   // normalizer entering the tile
    for (int c0 = 0; c0 < nC; c0 += GS_TILE) {
        const int nt = min(GS_TILE, nC - c0);
        for (int i = tid; i < nt; i += GS_THREADS) {
            const size_t t = tokh + (size_t)(c0 + i) * L + L - 1;
            sbl[i] = ws.b[t];
            sml[i] = ws.mloc[t];
        }
        __syncthreads();
        if (wave == 0) {
            const int run = (nt + 63) / 64;
            const int i0 = min(nt, lane * run), i1 = min(nt, i0 + run);
            double A = 0.0, B = -INFINITY;            // identity map
            for (int i = i0; i < i1; ++i) {
                A += sbl[i];
                B = fmax(B + sbl[i], sml[i]);
            }
            // inclusive scan of the lanes' maps, then shift to an exclusive one
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const double Ap = __shfl_up(A, off, 64), Bp = __shfl_up(B, off, 64);
                if (lane >= off) {
                    B = fmax(Bp + A, B);
                    A = Ap + A;
                }
            }
            double Ae = __shfl_up(A, 1, 64), Be = __shfl_up(B, 1, 64);
            if (lane == 0) { Ae = 0.0; Be = -INFINITY; }
            double mp = fmax(Ae + m_run, Be);
            for (int i = i0; i < i1; ++i) {
                smp[i] = mp;
                const double mL = fmax(sbl[i] + mp, sml[i]);
                salpha[i] = exp_arg(sbl[i] + mp - mL);
                srl[i] = exp_arg(sml[i] - mL);
                mp = mL;
            }
            if (lane == 63) smp[nt] = fmax(A + m_run, B);
        }
        __syncthreads();
        m_run = smp[nt];
        // per-token weights of this workgroup's share of the tile's tokens
        const int ntok = nt * L, per = (ntok + nparts - 1) / nparts;
        const int tlo = part * per, thi = min(ntok, tlo + per);
        for (int tb0 = tlo; tb0 < thi; tb0 += GS_THREADS * GS_BATCH) {
            double bt[GS_BATCH], ml[GS_BATCH];
            float wl[GS_BATCH];
#pragma unroll
            for (int u = 0; u < GS_BATCH; ++u) {
                const int t = tb0 + tid + GS_THREADS * u;
                if (t < thi) {
                    const size_t g = tokh + (size_t)c0 * L + t;
                    bt[u] = ws.b[g];
                    ml[u] = ws.mloc[g];
                    wl[u] = ws.wloc[g];
                }
            }
#pragma unroll
            for (int u = 0; u < GS_BATCH; ++u) {
                const int t = tb0 + tid + GS_THREADS * u;
                if (t < thi) {
                    const int ci = t / L;
                    const size_t g = tokh + (size_t)c0 * L + t;
                    const double mp = smp[ci];
                    const double mt = fmax(bt[u] + mp, ml[u]);
                    ws.a[g] = exp_arg(bt[u] + mp - mt);
                    ws.r[g] = exp_arg(ml[u] - mt);
                    ws.fl[g] = exp_arg(-mt);
                    ws.w[g] = srl[ci] * wl[u];
                    ws.alt[g] = salpha[ci];
                }
            }
        }
        if (part == 0)
            for (int i = tid; i < nt; i += GS_THREADS) ws.alpha[(size_t)bh * nC + c0 + i] = salpha[i];
        // normalizer entering each chunk: n' <- alpha n' + rl K^T w_loc, one key column per lane,
        // wave q over chunks [q0, q1) of the tile (workgroups past the key columns only
        // write per-token weights)
        if (part * GS_COLS >= dqk) continue;
        const int qrun = (nt + GS_WAVES - 1) / GS_WAVES;
        const int q0 = min(nt, wave * qrun), q1 = min(nt, q0 + qrun);
        const float* dnp = ws.dn + ((size_t)bh * nC + c0) * dqk + j;
        float* nep = ws.nent + ((size_t)bh * nC + c0) * dqk + j;
        float v = 0.0f, prod = 1.0f;
        for (int i0 = q0; i0 < q1; i0 += GS_BATCH) {
            float d[GS_BATCH];
#pragma unroll
            for (int e = 0; e < GS_BATCH; ++e)
                if (i0 + e < q1 && j < dqk) d[e] = dnp[(size_t)(i0 + e) * dqk];
#pragma unroll
            for (int e = 0; e < GS_BATCH; ++e)
                if (i0 + e < q1) {
                    v = salpha[i0 + e] * v + srl[i0 + e] * (j < dqk ? d[e] : 0.0f);
                    prod *= salpha[i0 + e];
                }
        }
        spart[wave][lane] = v;
        if (lane == 0) sprod[wave] = prod;
        __syncthreads();
        float nv = n_in;
        for (int w2 = 0; w2 < wave; ++w2) nv = sprod[w2] * nv + spart[w2][lane];
        for (int i0 = q0; i0 < q1; i0 += GS_BATCH) {
            float d[GS_BATCH];
#pragma unroll
            for (int e = 0; e < GS_BATCH; ++e)
                if (i0 + e < q1 && j < dqk) d[e] = dnp[(size_t)(i0 + e) * dqk];
#pragma unroll
            for (int e = 0; e < GS_BATCH; ++e)
                if (i0 + e < q1 && j < dqk) {
                    nep[(size_t)(i0 + e) * dqk] = nv;
                    nv = salpha[i0 + e] * nv + srl[i0 + e] * d[e];
                }
        }
        if (wave == GS_WAVES - 1) sfin[lane] = nv;
        __syncthreads();
        n_in = sfin[lane];
        __syncthreads();
    }
    if (wave == 0 && j < dqk) ws.nfin[(size_t)bh * dqk + j] = n_in;
    if (part == 0 && tid == 0) ws.mfin[bh] = (float)m_run;
}

// ---------------------------------------------------------------------------
// kernel 1c: the normalizer of every token
// ---------------------------------------------------------------------------
// den_t = r_t den_loc_t + a_t (q_t . n'_entering), in fp32: this is the quantity the
// retrieval divides by, and the one that cancels, so it is formed from exact bf16
// q and the fp32 normalizer state (no bf16 rounding of computed values).  What is
// stored is the inverted divisor 1 / max(|den_t|, exp(-m_t)), which the scan's
// output phase multiplies by.
constexpr int DEN_THREADS = 256;

template <int L>
__global__ __launch_bounds__(DEN_THREADS) void den_kernel(const bf16* __restrict__ q, Ws ws, int S, int Sx, int dqk)
{
    __shared__ __attribute__((aligned(16))) float sn[4096];
    const int c = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int nC = S / L;
    const float* ne = ws.nent + ((size_t)bh * nC + c) * dqk;
    for (int j = tid; j < dqk; j += DEN_THREADS) sn[j] = ne[j];
    __syncthreads();
    const size_t tok0 = (size_t)bh * S + (size_t)c * L;
    const int lp = tid & 15;
    // each 16-lane group takes rows tid/16 + 16 i; the rows' loads of one step are
    // issued together
    constexpr int RPT = L / (DEN_THREADS / 16);
    const bf16* qr = q + ((size_t)bh * Sx + (size_t)c * L + (tid >> 4)) * dqk;
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = 0.0f;
#pragma unroll 2
    for (int j0 = lp * 8; j0 < dqk; j0 += 128) {
        bf16x8 q8[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) q8[i] = *reinterpret_cast<const bf16x8*>(qr + (size_t)16 * i * dqk + j0);
        const f32x4 n0 = *reinterpret_cast<const f32x4*>(sn + j0);
        const f32x4 n1 = *reinterpret_cast<const f32x4*>(sn + j0 + 4);
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            acc[i] += (float)q8[i][0] * n0[0] + (float)q8[i][1] * n0[1] + (float)q8[i][2] * n0[2] +
                      (float)q8[i][3] * n0[3] + (float)q8[i][4] * n1[0] + (float)q8[i][5] * n1[1] +
                      (float)q8[i][6] * n1[2] + (float)q8[i][7] * n1[3];
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const float tot = row16_sum(acc[i]);
        if (lp == 0) {
            const size_t g = tok0 + (tid >> 4) + 16 * i;
            const float den = ws.r[g] * ws.den[g] + ws.a[g] * tot;
            ws.rden[g] = __builtin_amdgcn_rcpf(fmaxf(fabsf(den), ws.fl[g]));
        }
    }
}

// ---------------------------------------------------------------------------
// kernels 2a/2b: sequence segments (few heads, long sequences)
// ---------------------------------------------------------------------------
// Once gate_scan has put every per-token weight in the carried stabilization,
// the state after a run of chunks is affine in the state before it:
//   C'_end = A_g C'_start + dC_g,   A_g = prod_{c in g} alpha_c,
//   dC_g   = sum_{t in g} omega_t v_t k_t^T,  omega_t = w_t prod_{c in g, c > chunk(t)} alpha_c.
// seg_state_kernel forms dC_g of every segment but the last as one contraction
// over the segment's tokens (MFMA with fp32 accumulation; omega V split in bf16
// hi + lo as in the scan); seg_combine_kernel chains the segments.  The scan then
// runs every segment in parallel from its own entering state.
constexpr int SS_THREADS = 256;
constexpr int SS_P = SS_TILE + 16;     // LDS pitch (bf16) of the token-major tiles

template <int L>
__global__ __launch_bounds__(SS_THREADS) void seg_state_kernel(
    const bf16* __restrict__ k, const bf16* __restrict__ v, Ws ws, int S, int Sx, int dqk, int dv, int G)
{
    __shared__ __attribute__((aligned(16))) bf16 sk[L * SS_P];
    __shared__ __attribute__((aligned(16))) bf16 svh[L * SS_P];
    __shared__ __attribute__((aligned(16))) bf16 svl[L * SS_P];
    constexpr int UNITS = L * SS_TILE / 8;                  // 16-byte units of one tile
    constexpr int UPT = (UNITS + SS_THREADS - 1) / SS_THREADS;

    // a key width that is an odd multiple of 64 leaves the last tile's upper 64 keys
    // empty: they load as zeros and their waves skip the products and the store
    const int n_kt = (dqk + SS_TILE - 1) / SS_TILE;
    const int kt = blockIdx.x % n_kt, vt = blockIdx.x / n_kt;
    const int g = blockIdx.y / ws.sp, part = blockIdx.y % ws.sp, bh = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int ln = lane & 15, lg = lane >> 4;
    const int wr = wave >> 1, wc = wave & 1;                // 64 keys x 64 values per wave
    const int nC = S / L, nCs = nC / G, nCp = nCs / ws.sp;
    const int c_first = g * nCs + part * nCp;              // first chunk of this part
    const int key0 = kt * SS_TILE, val0 = vt * SS_TILE;
    const size_t tokh = (size_t)bh * S, tinh = (size_t)bh * Sx;

    // next chunk's K and V units, update weights of their rows and its alpha, in flight
    // while the current chunk is multiplied (chunks are walked last to first)
    bf16x8 rk[UPT], rv[UPT];
    float rw[UPT], ralpha = 1.0f;
    auto load = [&](int ci) {
        const int c = c_first + ci;
        const size_t t0 = tokh + (size_t)c * L, ti0 = tinh + (size_t)c * L;
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = tid + u * SS_THREADS;
            if (idx < UNITS) {
                const int row = idx / (SS_TILE / 8), c8 = 8 * (idx % (SS_TILE / 8));
                rk[u] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (key0 + c8 < dqk) rk[u] = *reinterpret_cast<const bf16x8*>(k + (ti0 + row) * dqk + key0 + c8);
                rv[u] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
                if (val0 + c8 < dv) rv[u] = *reinterpret_cast<const bf16x8*>(v + (ti0 + row) * dv + val0 + c8);
                rw[u] = ws.w[t0 + row];
            }
        }
        ralpha = ws.alpha[(size_t)bh * nC + c];
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0, 0, 0, 0};

    float A = 1.0f;          // product of alpha over the part's chunks after the current one
    const bool keys_in = key0 + 64 * wr < dqk;              // wave-uniform
    load(nCp - 1);
    for (int ci = nCp - 1; ci >= 0; --ci) {
        __syncthreads();     // previous tiles consumed
#pragma unroll
        for (int u = 0; u < UPT; ++u) {
            const int idx = tid + u * SS_THREADS;
            if (idx < UNITS) {
                const int row = idx / (SS_TILE / 8), c8 = 8 * (idx % (SS_TILE / 8));
                *reinterpret_cast<bf16x8*>(sk + row * SS_P + c8) = rk[u];
                bf16x8 xh, xl;
                split8w(rw[u] * A, rv[u], xh, xl);
                *reinterpret_cast<bf16x8*>(svh + row * SS_P + c8) = xh;
                *reinterpret_cast<bf16x8*>(svl + row * SS_P + c8) = xl;
            }
        }
        A *= ralpha;
        __syncthreads();
        if (ci > 0) load(ci - 1);
        if (!keys_in) continue;
#pragma unroll
        for (int kk = 0; kk < L / 32; ++kk) {
            const int trow = 32 * kk + 8 * lg + (ln >> 2);
            bf16x8 ka[4], vh[4], vl[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const bf16* kp = sk + trow * SS_P + 64 * wr + 16 * a + 4 * (ln & 3);
                ka[a] = cat(lds_read_tr(kp), lds_read_tr(kp + 4 * SS_P));
                const bf16* vp = svh + trow * SS_P + 64 * wc + 16 * a + 4 * (ln & 3);
                vh[a] = cat(lds_read_tr(vp), lds_read_tr(vp + 4 * SS_P));
                const bf16* vq = svl + trow * SS_P + 64 * wc + 16 * a + 4 * (ln & 3);
                vl[a] = cat(lds_read_tr(vq), lds_read_tr(vq + 4 * SS_P));
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc[a][b] = mfma(ka[a], vh[b], acc[a][b]);
                    acc[a][b] = mfma(ka[a], vl[b], acc[a][b]);
                }
        }
    }
    // the decay of the segment's chunks after this part
    float later = 1.0f;
    for (int c = c_first + nCp; c < (g + 1) * nCs; ++c) later *= ws.alpha[(size_t)bh * nC + c];
    // this part's share of dC_g: rows of the D layout are keys, columns are values
    float* dst = ws.cpart + (((size_t)bh * (G - 1) + g) * ws.sp + part) * (size_t)dv * dqk;
    if (!keys_in) return;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int col = val0 + 64 * wc + 16 * b + ln;
            if (col < dv)
                *reinterpret_cast<f32x4*>(dst + (size_t)col * dqk + key0 + 64 * wr + 16 * a + 4 * lg) = later * acc[a][b];
        }
}

constexpr int SC_THREADS = 256;
constexpr int SC_MAXG = 64;

// C'_start(g + 1) = A_g C'_start(g) + dC_g, with dC_g the sum of its parts in part
// order, into slots 1 .. G-1; slot 0 receives a copy of the initial state (or
// zero), so no segment reads the caller's buffer while another writes the final state.
__global__ __launch_bounds__(SC_THREADS) void seg_combine_kernel(Ws ws, int nC, int G, int dqk, int dv,
                                                                 const float* __restrict__ C0)
{
    __shared__ float sA[SC_MAXG];
    const int bh = blockIdx.y, tid = threadIdx.x;
    const int nCs = nC / G;
    if (tid < G - 1) {
        float prod = 1.0f;
        for (int ci = 0; ci < nCs; ++ci) prod *= ws.alpha[(size_t)bh * nC + tid * nCs + ci];
        sA[tid] = prod;
    }
    __syncthreads();
    const size_t per = (size_t)dv * dqk;
    const size_t e = ((size_t)blockIdx.x * SC_THREADS + tid) * 4;
    if (e >= per) return;
    f32x4 c = C0 ? *reinterpret_cast<const f32x4*>(C0 + (size_t)bh * per + e) : f32x4{0, 0, 0, 0};
    float* base = ws.cst + (size_t)bh * G * per + e;
    *reinterpret_cast<f32x4*>(base) = c;      // the first segment starts from slot 0
    const float* parts = ws.cpart + (size_t)bh * (G - 1) * ws.sp * per + e;
    for (int g = 0; g + 1 < G; ++g) {
        f32x4 d = *reinterpret_cast<const f32x4*>(parts + (size_t)g * ws.sp * per);
        for (int pp = 1; pp < ws.sp; ++pp) d += *reinterpret_cast<const f32x4*>(parts + ((size_t)g * ws.sp + pp) * per);
        c = sA[g] * c + d;
        *reinterpret_cast<f32x4*>(base + (size_t)(g + 1) * per) = c;
    }
}

// bf16 hi + lo split of two f32x4 state blocks into one B operand (8 key rows)

// ---------------------------------------------------------------------------
// kernel 2, pipelined form (chunks of 32 or 64 tokens)
// ---------------------------------------------------------------------------
// Same mathematics as chunk_scan, with every per-token weight and the entering
// normalizer precomputed by gate_scan, so the only sequential dependence left is
// the state itself.  Global loads run one step ahead of the MFMAs: while slab s
// is multiplied, slab s+1 (or slab 0 of the next chunk) is in flight into
// registers, and while chunk c is processed, chunk c+1's V tile, decayed scores,
// output-gate pre-activations and weights are in flight.  Q/K slabs are double
// buffered in LDS, so a slab costs one barrier; a chunk adds two (partial sums of
// Q C'^T over the key parts, and release of the chunk-level tiles).
template <int L_, int DQ_, int NC_, int NK_, int SB_, int MINB_, int CW_, bool RS_>
struct Scan2Cfg {
    static constexpr int L = L_, DQ = DQ_, NC = NC_, NK = NK_, SB = SB_, MINB = MINB_;
    static constexpr int CW = CW_;         // 16-column blocks per wave
    static constexpr bool RS = RS_;        // h rows stored 4 columns per lane after a quad transpose
    static constexpr int W = NC * NK, THREADS = 64 * W, TV = 16 * NC * CW;
    static constexpr int DP = DQ / NK, NS = DP / SB, SW = NK * SB;
    static constexpr int QP = SW + 4;      // Q pitch: row stride = 2 (mod 32) dwords
    static constexpr int KP = SW + 16;     // K pitch: row stride = 8 (mod 32) dwords
    static constexpr int VP = ((TV + 63) / 64) * 64 + 16;
    static constexpr int PP = L + 8, OP = TV + 4;
    static constexpr int LB = L / 16, SBB = SB / 16, NSB = DP / 16;
    static constexpr int RED = LB * (NK - 1) * NC * CW * 256;   // floats
    // staged 16-byte units
    static constexpr int U_Q = L * SW / 8, U_SLAB = 2 * U_Q;
    static constexpr int U_V = L * TV / 8, U_P = 2 * L * L / 8, U_O = L * TV / 4;
    static constexpr int U_SC = 3 * L / 4;   // a, r, rden
    static constexpr int U_CH = U_V + U_P + U_O + U_SC;
    static constexpr int NPS = (U_SLAB + THREADS - 1) / THREADS;
    static constexpr int NPC = (U_CH + THREADS - 1) / THREADS;
    static_assert(SW % 64 == 0 && SB % 32 == 0 && DP % SB == 0, "slab tiling");
    static_assert(LB % NK == 0 && L % 32 == 0 && L <= 64, "row blocks");
    static_assert(THREADS <= 1024, "workgroup too large");
};

template <class C>
struct alignas(16) Scan2Smem {
    alignas(16) bf16 q[2][C::L * C::QP];
    alignas(16) bf16 k[2][C::L * C::KP];
    alignas(16) bf16 v[C::L * C::VP];
    alignas(16) bf16 vwh[C::L * C::VP];  // (w / sigma') (.) V of the chunk, bf16 hi
    alignas(16) bf16 vwl[C::L * C::VP];  // and lo
    alignas(16) bf16 p[2][C::L * C::PP];
    alignas(16) float o[C::L * C::OP];
    alignas(16) float sc[3][C::L];       // a, r, rden
    // The partial retrievals of the key parts are exchanged through the K slab
    // buffer the chunk's last slab did not use when they fit there: every wave is
    // past the barrier of that slab, and the next chunk's first slab is stored
    // after the barrier that ends the chunk.  Otherwise they get their own array.
    static constexpr bool RED_IN_K = C::RED * sizeof(float) <= C::L * C::KP * sizeof(bf16);
    alignas(16) float red[RED_IN_K ? 4 : C::RED];
};

typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Per-thread loop over n 16-byte units of one staged region; `body(idx, u)` is
// called for idx = tid + u*THREADS < n with a compile-time u.
template <int THREADS, int N, int BASE, class F>
__device__ __forceinline__ void for_units(int tid, F&& body) {
#pragma unroll
    for (int u = 0; u < cdiv(N, THREADS); ++u) {
        const int idx = tid + u * THREADS;
        if ((N % THREADS == 0) || idx < N) body(idx, BASE + u);
    }
}

template <class C>
struct Pref {
    static constexpr int NQ = cdiv(C::U_Q, C::THREADS);      // Q units per thread
    static constexpr int NSL = 2 * NQ;                         // Q + K
    static constexpr int NV = cdiv(C::U_V, C::THREADS);
    static constexpr int NP = cdiv(C::U_P, C::THREADS);
    static constexpr int NO = cdiv(C::U_O, C::THREADS);
    static constexpr int NSC = cdiv(C::U_SC, C::THREADS);
    static constexpr int NCH = NV + NP + NO + NSC;
};

template <class C>
__device__ __forceinline__ void slab_load(f32x4 (&reg)[Pref<C>::NSL], int tid, const bf16* qh, const bf16* kh,
                                          size_t t0, int s) {
    constexpr int NQ = Pref<C>::NQ;
    auto src_off = [&](int idx) {
        const int row = idx / (C::SW / 8), c8 = 8 * (idx % (C::SW / 8));
        return (t0 + row) * C::DQ + s * C::SW + c8;
    };
    for_units<C::THREADS, C::U_Q, 0>(tid, [&](int idx, int u) {
        reg[u] = *reinterpret_cast<const f32x4*>(qh + src_off(idx));
    });
    for_units<C::THREADS, C::U_Q, NQ>(tid, [&](int idx, int u) {
        reg[u] = *reinterpret_cast<const f32x4*>(kh + src_off(idx));
    });
}

template <class C>
__device__ __forceinline__ void slab_store(const f32x4 (&reg)[Pref<C>::NSL], Scan2Smem<C>& sm, int buf, int tid) {
    constexpr int NQ = Pref<C>::NQ;
    for_units<C::THREADS, C::U_Q, 0>(tid, [&](int idx, int u) {
        const int row = idx / (C::SW / 8), c8 = 8 * (idx % (C::SW / 8));
        f32x2* d = reinterpret_cast<f32x2*>(sm.q[buf] + row * C::QP + c8);   // 8-byte aligned rows
        d[0] = f32x2{reg[u][0], reg[u][1]};
        d[1] = f32x2{reg[u][2], reg[u][3]};
    });
    for_units<C::THREADS, C::U_Q, NQ>(tid, [&](int idx, int u) {
        const int row = idx / (C::SW / 8), c8 = 8 * (idx % (C::SW / 8));
        *reinterpret_cast<f32x4*>(sm.k[buf] + row * C::KP + c8) = reg[u];
    });
}

struct ChunkSrc {
    const bf16* v; const bf16* P; const float* o;
    const float* sc;     // a of the chunk's first token; r, rden, fl, w, alt follow at stride hs
    size_t hs;
    int vcols;           // valid value columns of the tile
};

template <class C>
__device__ __forceinline__ void chunk_load(f32x4 (&reg)[Pref<C>::NCH], float (&wrow)[Pref<C>::NV], float& alpha,
                                           int tid, const ChunkSrc& cs, int dv) {
    using PF = Pref<C>;
    for_units<C::THREADS, C::U_V, 0>(tid, [&](int idx, int u) {
        const int row = idx / (C::TV / 8), col = 8 * (idx % (C::TV / 8));
        reg[u] = (col < cs.vcols) ? *reinterpret_cast<const f32x4*>(cs.v + (size_t)row * dv + col) : f32x4{0, 0, 0, 0};
        wrow[u] = cs.sc[4 * cs.hs + row];          // update weight w of the unit's token
    });
    alpha = cs.sc[5 * cs.hs];                      // the chunk's decay (repeated per token)
    for_units<C::THREADS, C::U_P, PF::NV>(tid, [&](int idx, int u) {
        reg[u] = *reinterpret_cast<const f32x4*>(cs.P + 8 * idx);
    });
    for_units<C::THREADS, C::U_O, PF::NV + PF::NP>(tid, [&](int idx, int u) {
        const int row = idx / (C::TV / 4), col = 4 * (idx % (C::TV / 4));
        reg[u] = (col < cs.vcols) ? *reinterpret_cast<const f32x4*>(cs.o + (size_t)row * dv + col) : f32x4{0, 0, 0, 0};
    });
    for_units<C::THREADS, C::U_SC, PF::NV + PF::NP + PF::NO>(tid, [&](int idx, int u) {
        const int arr = idx / (C::L / 4), i4 = idx % (C::L / 4);
        reg[u] = *reinterpret_cast<const f32x4*>(cs.sc + arr * cs.hs + 4 * i4);
    });
}

// inv_sig = 1 / sigma' of the chunk: the V units are also stored as (w / sigma') (.) V,
// split into bf16 hi + lo, the B operand of the state update
template <class C>
__device__ __forceinline__ void chunk_store(const f32x4 (&reg)[Pref<C>::NCH], const float (&wrow)[Pref<C>::NV],
                                            float inv_sig, Scan2Smem<C>& sm, int tid) {
    using PF = Pref<C>;
    for_units<C::THREADS, C::U_V, 0>(tid, [&](int idx, int u) {
        const int row = idx / (C::TV / 8), col = 8 * (idx % (C::TV / 8));
        *reinterpret_cast<f32x4*>(sm.v + row * C::VP + col) = reg[u];
        const bf16x8 vb = __builtin_bit_cast(bf16x8, reg[u]);
        bf16x8 h, l;
        split8w(wrow[u] * inv_sig, vb, h, l);
        *reinterpret_cast<bf16x8*>(sm.vwh + row * C::VP + col) = h;
        *reinterpret_cast<bf16x8*>(sm.vwl + row * C::VP + col) = l;
    });
    for_units<C::THREADS, C::U_P, PF::NV>(tid, [&](int idx, int u) {
        const int half = idx / (C::L * C::L / 8), rem = idx % (C::L * C::L / 8);
        const int row = rem / (C::L / 8), col = 8 * (rem % (C::L / 8));
        *reinterpret_cast<f32x4*>(sm.p[half] + row * C::PP + col) = reg[u];
    });
    for_units<C::THREADS, C::U_O, PF::NV + PF::NP>(tid, [&](int idx, int u) {
        const int row = idx / (C::TV / 4), col = 4 * (idx % (C::TV / 4));
        *reinterpret_cast<f32x4*>(sm.o + row * C::OP + col) = reg[u];
    });
    for_units<C::THREADS, C::U_SC, PF::NV + PF::NP + PF::NO>(tid, [&](int idx, int u) {
        const int arr = idx / (C::L / 4), i4 = idx % (C::L / 4);
        *reinterpret_cast<f32x4*>(&sm.sc[arr][4 * i4]) = reg[u];
    });
}

// The mLSTM block's epilogue ("xLSTM: Extended Long Short-Term Memory", Figure 10
// and its caption) applied to whole rows of h in the scan's output phase:
// y = (gn_w (.) (h - mean) / sqrt(var + eps) + gn_b + skip_w (.) x) (.) act(z), the
// mean and population variance over the head's d_v channels of the row.
struct EpiArgs {
    const bf16* x; const bf16* z;
    const float* gw; const float* gb; const float* sw;   // [NH][d_v]
    float eps; int act; int NH;
};

template <class C, bool EPI = false>
__global__ __launch_bounds__(C::THREADS, C::MINB) void chunk_scan2_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const float* __restrict__ o_pre, Ws ws, int S, int Sx, int G, int dv, int n_vt, int remap,
    const float* __restrict__ C0,
    bf16* __restrict__ h, float* __restrict__ Cout, float* __restrict__ nout, float* __restrict__ mout,
    EpiArgs ep)
{
    constexpr int L = C::L, DQ = C::DQ, NC = C::NC, NK = C::NK, SB = C::SB, CW = C::CW;
    constexpr int THREADS = C::THREADS, TV = C::TV, NS = C::NS;
    constexpr int QP = C::QP, KP = C::KP, VP = C::VP, PP = C::PP, OP = C::OP;
    constexpr int LB = C::LB, SBB = C::SBB, NSB = C::NSB;
    // Lazy decay: the registers hold C^ = C' / sigma; each chunk's decay alpha is
    // folded into sigma and into the weights of the update (w / sigma) and of the
    // retrieval (a sigma), and the registers are rescaled only when sigma would
    // leave the range where 1/sigma is comfortably finite.
    constexpr float SIGMA_MIN = 0x1p-60f;
    __shared__ Scan2Smem<C> sm;

    int wg = blockIdx.x;
    if (remap) {
        const int G = gridDim.x;
        wg = (wg % 8) * (G / 8) + wg / 8;
    }
    // workgroup -> (head, sequence segment, value tile)
    const int bh = wg / (G * n_vt), seg = (wg / n_vt) % G, vt = wg % n_vt;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int cb = wave % NC, kq = wave / NC;
    const int ln = lane & 15, lg = lane >> 4;
    // this wave's CW column blocks: tile columns 16 * (CW * cb + x), x < CW
    const int tcol = 16 * CW * cb;
    const int vcol = vt * TV + tcol;
    bool act[CW];
#pragma unroll
    for (int x = 0; x < CW; ++x) act[x] = vcol + 16 * x < dv;
    const bool active = act[0];
    const int nC = S / L / G;                      // chunks of this segment

    const size_t tokh = (size_t)bh * S + (size_t)seg * (S / G);    // workspace token index
    const size_t tinh = (size_t)bh * Sx + (size_t)seg * (S / G);   // input / output token index
    // state entering the segment: the caller's (or zero) for the first, else the chained one
    const float* Cin = G == 1 ? (C0 ? C0 + (size_t)bh * dv * DQ : nullptr)
                              : ws.cst + ((size_t)bh * G + seg) * (size_t)dv * DQ;
    const bf16* qh = q + tinh * DQ;
    const bf16* kh = k + tinh * DQ;
    bf16* hh = h + tinh * dv;

    auto chunk_src = [&](int c) {
        ChunkSrc cs;
        const size_t t0 = (size_t)c * L;
        cs.v = v + (tinh + t0) * dv + vt * TV;
        cs.P = ws.P + 2 * (tokh + t0) * L;
        cs.o = o_pre + (tinh + t0) * dv + vt * TV;
        cs.sc = ws.a + tokh + t0;
        cs.hs = ws.hs;
        cs.vcols = min(TV, dv - vt * TV);
        return cs;
    };

    // state: st[x][jb] holds key rows j = s*SW + kq*SB + 16*jj + 4*lg + i (jb = s*SBB + jj), value
    // column vcol + 16x + ln.  A slab is NK*SB consecutive keys, so its rows are read as
    // whole cache lines, and key part kq takes its SB columns.
    f32x4 st[CW][NSB];
#pragma unroll
    for (int x = 0; x < CW; ++x)
#pragma unroll
        for (int jb = 0; jb < NSB; ++jb) {
            st[x][jb] = f32x4{0, 0, 0, 0};
            if (Cin && act[x])
                st[x][jb] = *reinterpret_cast<const f32x4*>(
                    Cin + (size_t)(vcol + 16 * x + ln) * DQ + (jb / SBB) * C::SW + kq * SB + 16 * (jb % SBB) + 4 * lg);
        }

    f32x4 rs[Pref<C>::NSL], rc[Pref<C>::NCH];
    float rw[Pref<C>::NV], ralpha;
    chunk_load<C>(rc, rw, ralpha, tid, chunk_src(0), dv);
    slab_load<C>(rs, tid, qh, kh, 0, 0);
    float sigma = 1.0f;

    // the block epilogue's per-channel parameters of this lane's columns, and the skip
    // inputs and gate pre-activations of the rows this wave finishes, loaded a chunk
    // ahead of the output phase that uses them
    constexpr int NOB = LB / NK;
    bf16 xr[NOB][CW][4], zr[NOB][CW][4];
    // element offset of this lane's (row 4 lg + 16 (kq + NK j) + i, column 16 x + ln)
    // within a chunk's rows, 32-bit: the chunk base is the only 64-bit address
    auto rc_off = [&](int j, int x, int i) {
        return (16 * (kq + NK * j) + 4 * lg + i) * dv + min(vcol + 16 * x, dv - 16) + ln;
    };
    auto load_xz = [&](int cc) {
        const bf16* xb = ep.x + (tinh + (size_t)cc * L) * dv;
        const bf16* zb = ep.z + (tinh + (size_t)cc * L) * dv;
#pragma unroll
        for (int j = 0; j < NOB; ++j)
#pragma unroll
            for (int x = 0; x < CW; ++x)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xr[j][x][i] = xb[rc_off(j, x, i)];
                    zr[j][x][i] = zb[rc_off(j, x, i)];
                }
    };
    float egw[CW] = {}, egb[CW] = {}, esw[CW] = {};
    // Rows of chunk c are finished during chunk c + 1: the row sums written in chunk
    // c's output phase are complete after its last barrier, so epi_mean runs at the
    // top of chunk c + 1 and writes the centered sums, which are complete after the
    // next slab barrier, where epi_out normalizes, gates and stores the rows (beside
    // that slab's products).  No barrier is added to the chunk.
    __shared__ float epi[EPI ? 2 : 1][2][EPI ? L : 1][EPI ? NC : 1];  // [chunk parity][sums, centered][row][wave]
    f32x4 yyp[NOB][CW];
    float mup[NOB][4];
    const float inv_dv = 1.0f / (float)dv;
    auto epi_mean = [&](int cc) {
#pragma unroll
        for (int j = 0; j < NOB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * (kq + NK * j) + 4 * lg + i;
                float t = 0.0f;
#pragma unroll
                for (int c2 = 0; c2 < NC; ++c2) t += epi[cc & 1][0][row][c2];
                mup[j][i] = t * inv_dv;
                float s2 = 0.0f;
#pragma unroll
                for (int x = 0; x < CW; ++x)
                    if (act[x]) {
                        const float d = yyp[j][x][i] - mup[j][i];
                        s2 += d * d;
                    }
                s2 = row16_sum(s2);
                if (ln == 0) epi[cc & 1][1][row][cb] = s2;
            }
    };
    auto epi_out = [&](int cc) {
        if (active) {
            bf16* yb = hh + (size_t)cc * L * dv;
#pragma unroll
            for (int j = 0; j < NOB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * (kq + NK * j) + 4 * lg + i;
                    float t = 0.0f;
#pragma unroll
                    for (int c2 = 0; c2 < NC; ++c2) t += epi[cc & 1][1][row][c2];
                    const float rs = __builtin_amdgcn_rsqf(t * inv_dv + ep.eps);
#pragma unroll
                    for (int x = 0; x < CW; ++x) {
                        if (!act[x]) continue;
                        const float xv = (float)xr[j][x][i], zv = (float)zr[j][x][i];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-zv));
                        const float g = ep.act ? zv * sg : sg;
                        const float yo = (egw[x] * (yyp[j][x][i] - mup[j][i]) * rs + egb[x] + esw[x] * xv) * g;
                        yb[rc_off(j, x, i)] = (bf16)yo;
                    }
                }
        }
        load_xz(min(cc + 1, nC - 1));   // the rows finished during the next chunk
    };
    if constexpr (EPI) {
        load_xz(0);
        const int hd = bh % ep.NH;
#pragma unroll
        for (int x = 0; x < CW; ++x) {
            const size_t pc = (size_t)hd * dv + min(vcol + 16 * x, dv - 16) + ln;
            egw[x] = ep.gw[pc];
            egb[x] = ep.gb[pc];
            esw[x] = ep.sw[pc];
        }
    }

    for (int c = 0; c < nC; ++c) {
        const size_t t0 = (size_t)c * L;
        // sigma' after this chunk's decay; the registers are rescaled instead when
        // it would leave the comfortable range (every thread takes the same decision)
        const float cand = sigma * ralpha;
        const bool rescale = cand < SIGMA_MIN;
        const float st_scale = rescale ? cand : 1.0f;
        const float sig_new = rescale ? 1.0f : cand;
        chunk_store<C>(rc, rw, 1.0f / sig_new, sm, tid);
        f32x4 acc_inter[LB][CW];
#pragma unroll
        for (int tb = 0; tb < LB; ++tb)
#pragma unroll
            for (int x = 0; x < CW; ++x) acc_inter[tb][x] = f32x4{0, 0, 0, 0};
        bf16x8 vwh[CW][L / 32], vwl[CW][L / 32];

#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int buf = (c * NS + s) & 1;
            if constexpr (EPI) {
                if (s == 0 && c > 0) epi_mean(c - 1);
            }
            slab_store<C>(rs, sm, buf, tid);
            lds_barrier();
            // next loads in flight while this slab is multiplied
            if (s + 1 < NS) slab_load<C>(rs, tid, qh, kh, t0, s + 1);
            else if (c + 1 < nC) slab_load<C>(rs, tid, qh, kh, t0 + L, 0);
            if constexpr (EPI) {
                if (s == 0 && c > 0) epi_out(c - 1);
            }
            if (active) {
                if (s == 0) {
                    // this wave's columns of (w / sigma') (.) V, hi and lo, as B operands
#pragma unroll
                    for (int kk = 0; kk < L / 32; ++kk)
#pragma unroll
                        for (int x = 0; x < CW; ++x) {
                            const int vrow = (32 * kk + 8 * lg + (ln >> 2)) * VP + tcol + 16 * x + 4 * (ln & 3);
                            vwh[x][kk] = cat(lds_read_tr(sm.vwh + vrow), lds_read_tr(sm.vwh + vrow + 4 * VP));
                            vwl[x][kk] = cat(lds_read_tr(sm.vwl + vrow), lds_read_tr(sm.vwl + vrow + 4 * VP));
                        }
                }
                __builtin_amdgcn_sched_barrier(0);
                // The slab's operands are read from LDS before the products that use
                // them, and the K operands of the update stream in while the
                // retrieval multiplies, so the matrix pipe does not wait on LDS
                // latency operand by operand.
                constexpr int KQ = SB / 32, KU = L / 32;
                bf16x8 qa[KQ][LB], ka[KU][SBB];
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk)
#pragma unroll
                    for (int tb = 0; tb < LB; ++tb) {
                        const bf16* qp = sm.q[buf] + (16 * tb + ln) * QP + kq * SB + 32 * kk + 4 * lg;
                        qa[kk][tb] = cat(*reinterpret_cast<const bf16x4*>(qp), *reinterpret_cast<const bf16x4*>(qp + 16));
                    }
#pragma unroll
                for (int kk = 0; kk < KU; ++kk)
#pragma unroll
                    for (int jb = 0; jb < SBB; ++jb) {
                        const bf16* kp = sm.k[buf] + (32 * kk + 8 * lg + (ln >> 2)) * KP + kq * SB + 16 * jb + 4 * (ln & 3);
                        ka[kk][jb] = cat(lds_read_tr(kp), lds_read_tr(kp + 4 * KP));
                    }
                // inter-chunk retrieval: acc_inter += Q[:, slab] (C^_hi + C^_lo)^T[slab, cols];
                // each Q operand serves all CW column blocks
#pragma unroll
                for (int kk = 0; kk < KQ; ++kk) {
                    bf16x8 bhi[CW], blo[CW];
#pragma unroll
                    for (int x = 0; x < CW; ++x)
                        split8(st[x][s * SBB + 2 * kk], st[x][s * SBB + 2 * kk + 1], bhi[x], blo[x]);
#pragma unroll
                    for (int tb = 0; tb < LB; ++tb)
#pragma unroll
                        for (int x = 0; x < CW; ++x) {
                            acc_inter[tb][x] = mfma(qa[kk][tb], bhi[x], acc_inter[tb][x]);
                            acc_inter[tb][x] = mfma(qa[kk][tb], blo[x], acc_inter[tb][x]);
                        }
                }
                // state update: C^[slab] += K[:, slab]^T ((w / sigma') V)_{hi+lo}
#pragma unroll
                for (int x = 0; x < CW; ++x)
#pragma unroll
                    for (int jb = 0; jb < SBB; ++jb) st[x][s * SBB + jb] *= st_scale;
#pragma unroll
                for (int kk = 0; kk < KU; ++kk)
#pragma unroll
                    for (int jb = 0; jb < SBB; ++jb)
#pragma unroll
                        for (int x = 0; x < CW; ++x) {
                            st[x][s * SBB + jb] = mfma(ka[kk][jb], vwh[x][kk], st[x][s * SBB + jb]);
                            st[x][s * SBB + jb] = mfma(ka[kk][jb], vwl[x][kk], st[x][s * SBB + jb]);
                        }
                // instruction order: all Q reads, then the K reads one by one between
                // the retrieval products, then the remaining products
                constexpr int NQR = KQ * LB, NKR = 2 * KU * SBB;
                constexpr int NMI = 2 * KQ * LB * CW, NMU = 2 * KU * SBB * CW;
                static_assert(NMI >= NKR, "enough retrieval products to cover the K reads");
                __builtin_amdgcn_sched_group_barrier(0x100, NQR, 0);
#pragma unroll
                for (int i = 0; i < NKR; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NMI + NMU - NKR, 0);
            }
            // the next chunk's tiles are requested after this slab's products are issued
            if (s == NS - 1 && c + 1 < nC) {
                __builtin_amdgcn_sched_barrier(0);
                chunk_load<C>(rc, rw, ralpha, tid, chunk_src(c + 1), dv);
            }
        }

        // --- partial sums over key parts, then the rows each part owns --------
        float* red = Scan2Smem<C>::RED_IN_K ? reinterpret_cast<float*>(sm.k[1 - ((c * NS + NS - 1) & 1)]) : sm.red;
        if (NK > 1 && active) {
#pragma unroll
            for (int tb = 0; tb < LB; ++tb) {
                const int owner = tb % NK;
                if (owner == kq) continue;
                const int slot = kq < owner ? kq : kq - 1;
#pragma unroll
                for (int x = 0; x < CW; ++x)
                    *reinterpret_cast<f32x4*>(red + ((((tb * (NK - 1) + slot) * NC + cb) * CW + x) * 256 + lane * 4)) =
                        acc_inter[tb][x];
            }
        }
        lds_barrier();
        if constexpr (EPI) {
            // Whole rows of the head are in this workgroup (one value tile): each wave
            // keeps h of its row blocks in registers and puts the row sums over its
            // columns in LDS; the next chunk finishes these rows (epi_mean, epi_out).
            f32x4 (&yy)[NOB][CW] = yyp;
#pragma unroll
            for (int j = 0; j < NOB; ++j)
#pragma unroll
                for (int x = 0; x < CW; ++x) yy[j][x] = f32x4{0, 0, 0, 0};
            // row blocks walked with compile-time indices (this wave's are tb = kq + NK j)
#pragma unroll
            for (int tb = 0; tb < LB; ++tb) {
                if (tb % NK != kq || !active) continue;
                const int j = tb / NK;
                f32x4 inter[CW], intra[CW];
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    inter[x] = acc_inter[tb][x];
#pragma unroll
                    for (int sl = 0; sl < NK - 1; ++sl)
                        inter[x] += *reinterpret_cast<const f32x4*>(
                            red + ((((tb * (NK - 1) + sl) * NC + cb) * CW + x) * 256 + lane * 4));
                    intra[x] = f32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int kk = 0; kk <= (16 * tb + 15) / 32; ++kk) {
                    const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(sm.p[0] + (16 * tb + ln) * PP + 32 * kk + 8 * lg);
                    const bf16x8 alo = *reinterpret_cast<const bf16x8*>(sm.p[1] + (16 * tb + ln) * PP + 32 * kk + 8 * lg);
#pragma unroll
                    for (int x = 0; x < CW; ++x) {
                        const bf16* vb = sm.v + (32 * kk + 8 * lg + (ln >> 2)) * VP + tcol + 16 * x + 4 * (ln & 3);
                        const bf16x8 bop = cat(lds_read_tr(vb), lds_read_tr(vb + 4 * VP));
                        intra[x] = mfma(ahi, bop, intra[x]);
                        intra[x] = mfma(alo, bop, intra[x]);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tau = 16 * tb + 4 * lg + i;
                    const float aa = sm.sc[0][tau] * sigma, ra = sm.sc[1][tau], rden = sm.sc[2][tau];
#pragma unroll
                    for (int x = 0; x < CW; ++x) {
                        if (!act[x]) continue;
                        const float num = ra * intra[x][i] + aa * inter[x][i];
                        const float og = __builtin_amdgcn_rcpf(1.0f + __expf(-sm.o[tau * OP + tcol + 16 * x + ln]));
                        yy[j][x][i] = og * num * rden;
                    }
                }
            }
            // row sums over this wave's columns (the 16 lanes of a lane group hold one row)
#pragma unroll
            for (int j = 0; j < NOB; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float s1 = 0.0f;
#pragma unroll
                    for (int x = 0; x < CW; ++x) s1 += yy[j][x][i];
                    s1 = row16_sum(s1);
                    if (ln == 0) epi[c & 1][0][16 * (kq + NK * j) + 4 * lg + i][cb] = s1;
                }
        } else if (active) {
#pragma unroll
            for (int tb = 0; tb < LB; ++tb) {
                if (tb % NK != kq) continue;
                f32x4 inter[CW], intra[CW];
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    inter[x] = acc_inter[tb][x];
#pragma unroll
                    for (int sl = 0; sl < NK - 1; ++sl)
                        inter[x] += *reinterpret_cast<const f32x4*>(
                            red + ((((tb * (NK - 1) + sl) * NC + cb) * CW + x) * 256 + lane * 4));
                    intra[x] = f32x4{0, 0, 0, 0};
                }
#pragma unroll
                for (int kk = 0; kk <= (16 * tb + 15) / 32; ++kk) {
                    const bf16x8 ahi = *reinterpret_cast<const bf16x8*>(sm.p[0] + (16 * tb + ln) * PP + 32 * kk + 8 * lg);
                    const bf16x8 alo = *reinterpret_cast<const bf16x8*>(sm.p[1] + (16 * tb + ln) * PP + 32 * kk + 8 * lg);
#pragma unroll
                    for (int x = 0; x < CW; ++x) {
                        const bf16* vb = sm.v + (32 * kk + 8 * lg + (ln >> 2)) * VP + tcol + 16 * x + 4 * (ln & 3);
                        const bf16x8 bop = cat(lds_read_tr(vb), lds_read_tr(vb + 4 * VP));
                        intra[x] = mfma(ahi, bop, intra[x]);
                        intra[x] = mfma(alo, bop, intra[x]);
                    }
                }
                f32x4 y[CW];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tau = 16 * tb + 4 * lg + i;
                    const float aa = sm.sc[0][tau] * sigma, ra = sm.sc[1][tau], rden = sm.sc[2][tau];
#pragma unroll
                    for (int x = 0; x < CW; ++x) {
                        const float num = ra * intra[x][i] + aa * inter[x][i];
                        const float og = __builtin_amdgcn_rcpf(1.0f + __expf(-sm.o[tau * OP + tcol + 16 * x + ln]));
                        y[x][i] = og * num * rden;
                    }
                }
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    if (!act[x]) continue;
                    if constexpr (C::RS) {
                        // one 8-byte store per lane: row 16 tb + 4 lg + (ln & 3), 4 columns
                        const f32x4 t = quad_transpose(y[x], ln & 3);
                        *reinterpret_cast<bf16x4*>(hh + (t0 + 16 * tb + 4 * lg + (ln & 3)) * dv + vcol + 16 * x +
                                                   4 * (ln >> 2)) = bf16x4{(bf16)t[0], (bf16)t[1], (bf16)t[2], (bf16)t[3]};
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            hh[(t0 + 16 * tb + 4 * lg + i) * dv + vcol + 16 * x + ln] = (bf16)y[x][i];
                    }
                }
            }
        }
        sigma = sig_new;
        lds_barrier();
    }
    if constexpr (EPI) {
        epi_mean(nC - 1);
        lds_barrier();
        epi_out(nC - 1);
    }

    if (seg != G - 1) return;
#pragma unroll
    for (int x = 0; x < CW; ++x) {
        if (!act[x]) continue;
#pragma unroll
        for (int jb = 0; jb < NSB; ++jb)
            *reinterpret_cast<f32x4*>(Cout + ((size_t)bh * dv + vcol + 16 * x + ln) * DQ + (jb / SBB) * C::SW + kq * SB +
                                      16 * (jb % SBB) + 4 * lg) =
                st[x][jb] * sigma;
    }
    if (vt == 0) {
        for (int j = tid; j < DQ; j += THREADS) nout[(size_t)bh * DQ + j] = ws.nfin[(size_t)bh * DQ + j];
        if (tid == 0) mout[bh] = ws.mfin[bh];
    }
}

// ---------------------------------------------------------------------------
// kernel 2, streaming form (64-token chunks)
// ---------------------------------------------------------------------------
// Every wave owns all TV value columns of the tile and DP = DQ/NK key rows of C'^T,
// so each element of Q and K is needed by exactly one wave: both come from global
// memory (L2) straight into that wave's MFMA operand registers, in the
// operand-ordered copies chunk_prep writes (one contiguous 1 KB load per operand
// block), and the key dimension needs no LDS staging and no barriers.  Per chunk a
// wave makes two sweeps over its key rows: the retrieval Q C'^T of the state
// entering the chunk, then the update C' += K^T ((w / sigma') V).  The partial
// retrievals of the NK key parts go to LDS; each wave finishes the output rows of
// the blocks it owns during the next chunk's retrieval sweep, so the one barrier
// per chunk sits at its end.  The chunk's V tile and (w / sigma') (.) V, split into
// bf16 hi + lo, are formed once per workgroup at the end of the previous chunk.
//
// Key order.  The state block pair (2s, 2s+1) of a wave covers its key rows
// 32s .. 32s+31; block 2s + jt holds key 32s + 8(r/4) + 4jt + r%4 in accumulator
// row r.  Lane l then holds keys 32s + 8(l/16) .. + 7 of the pair (rows 4(l/16)+i
// of both blocks), which is exactly the B operand layout of the retrieval against
// 8 consecutive keys of a Q row, and the update's A operand row r of block 2s + jt
// is the token-contiguous K^T row of that key.
//
// Loads are branch free (indices past the last chunk are clamped to it) and each
// step's prefetch is pinned before its products, so the compiler can count the
// loads in flight instead of draining them at every step.
template <int DQ_, int NK_, int CW_, int MINB_, int PD_, bool OP_ = true>
struct Scan4Cfg {
    static constexpr int L = 64, DQ = DQ_, NK = NK_, CW = CW_, MINB = MINB_;
    static constexpr bool OUT_PREFETCH = OP_;   // output operands loaded a chunk ahead
    static constexpr int PD = PD_;              // operand steps in flight ahead of the one multiplied
    static constexpr int THREADS = 64 * NK, TV = 16 * CW;
    static constexpr int DP = DQ / NK;          // key rows per wave
    static constexpr int NS = DP / 32;          // 32-key steps per wave
    static constexpr int LB = L / 16;           // 16-row blocks of the chunk
    static constexpr int NB = LB * CW;          // output blocks of the tile
    static constexpr int NOWN = (NB + NK - 1) / NK;
    // tile pitch (bf16): 16 or 48 mod 64, so that the 4 rows of a transposing read
    // start 8 or 24 banks apart and hit distinct banks
    static constexpr int VP = (TV % 64 == 16 || TV % 64 == 48) ? TV : TV + 16;
    static constexpr int U_V = L * TV / 8;      // 16-byte units of the V tile
    static constexpr int NPV = (U_V + THREADS - 1) / THREADS;
    static constexpr int RED = NB * (NK - 1) * 256;   // floats of one partial-sum buffer (owners keep theirs)
    static constexpr size_t TILES = 7 * (size_t)L * VP * 2;
    static_assert(MINB * (TILES + 2 * (size_t)RED * 4) <= 160 * 1024, "LDS");
    static_assert(DQ % NK == 0 && DP % 32 == 0, "key parts of whole 32-key steps");
    static_assert(THREADS <= 1024, "workgroup too large");
    static_assert(PD >= 1 && PD <= 2 * NS, "prefetch depth within one chunk's steps");
};

// raw buffer loads (16 bytes): descriptor word 3 of an untyped buffer on gfx9-family
// parts; reads past the descriptor's byte count return zeros
constexpr int BUF_DWORD3 = 0x00020000;
__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

template <class C>
struct alignas(16) Scan4Smem {
    alignas(16) bf16 v[3][C::L * C::VP];     // V tile of the chunk
    alignas(16) bf16 vwh[2][C::L * C::VP];   // (w / sigma') (.) V, bf16 hi
    alignas(16) bf16 vwl[2][C::L * C::VP];   // and lo
    alignas(16) float red[2][C::RED];
};

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void chunk_scan4_kernel(
    const bf16* __restrict__ v,
    const float* __restrict__ o_pre, Ws ws, int S, int Sx, int G, int dv, int n_vt, int remap,
    const float* __restrict__ C0,
    bf16* __restrict__ h, float* __restrict__ Cout, float* __restrict__ nout, float* __restrict__ mout)
{
    constexpr int L = C::L, DQ = C::DQ, NK = C::NK, CW = C::CW;
    constexpr int THREADS = C::THREADS, TV = C::TV, DP = C::DP, NS = C::NS;
    constexpr int LB = C::LB, NB = C::NB, VP = C::VP, PD = C::PD;
    constexpr float SIGMA_MIN = 0x1p-60f;
    __shared__ Scan4Smem<C> sm;

    int wg = blockIdx.x;
    if (remap) {
        const int NG = gridDim.x;
        wg = (wg % 8) * (NG / 8) + wg / 8;
    }
    const int bh = wg / (G * n_vt), seg = (wg / n_vt) % G, vt = wg % n_vt;
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int ln = lane & 15, lg = lane >> 4;
    const int vcol = vt * TV;
    const int vcols = min(TV, dv - vcol);
    const int nC = S / L / G;
    const int nCh = S / L;

    const size_t tokh = (size_t)bh * S + (size_t)seg * (S / G);
    const size_t tinh = (size_t)bh * Sx + (size_t)seg * (S / G);
    const size_t ch0 = (size_t)bh * nCh + (size_t)seg * nC;       // global chunk index of chunk 0
    const float* Cin = G == 1 ? (C0 ? C0 + (size_t)bh * dv * DQ : nullptr)
                              : ws.cst + ((size_t)bh * G + seg) * (size_t)dv * DQ;
    const int kw = wave * DP;                                      // this wave's first key row
    // Q and K^T come in the operand-ordered copies chunk_prep writes: the fragment of
    // 32-key step ks and block f of chunk c is 1 KB at ((c * DQ/32 + ks) * 4 + f) KB of
    // the segment, lane l's 16 bytes at l * 16.  Q block tb: row 16 tb + ln, keys
    // 32 ks + 8 lg .. + 7; K^T block 2 jt + kk: key 32 ks + 8 (ln / 4) + 4 jt + ln % 4,
    // tokens 32 kk + 8 lg .. + 7.  Buffer descriptors keep every offset but the lane's
    // in scalar registers.
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ws.qs + tokh * DQ), (short)0, (int)((size_t)nC * L * DQ * 2), BUF_DWORD3);
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ws.ks + tokh * DQ), (short)0, (int)((size_t)nC * L * DQ * 2), BUF_DWORD3);
    const int vl = lane * 16;
    constexpr int KSTEPS = DQ / 32;

    // state: st[x][2s + jt][i] = C^[key kw + 32s + 8lg + 4jt + i][column vcol + 16x + ln]
    f32x4 st[CW][2 * NS];
#pragma unroll
    for (int x = 0; x < CW; ++x)
#pragma unroll
        for (int b = 0; b < 2 * NS; ++b) {
            st[x][b] = f32x4{0, 0, 0, 0};
            if (Cin && 16 * x < vcols)
                st[x][b] = *reinterpret_cast<const f32x4*>(
                    Cin + (size_t)(vcol + 16 * x + ln) * DQ + kw + 32 * (b / 2) + 8 * lg + 4 * (b % 2));
        }

    // operand stream: step t < NS of a chunk is Q step t, NS <= t < 2NS is K^T step
    // t - NS; PD steps are in flight while one is multiplied
    auto load_step = [&](bf16x8 (&r)[4], int c, int t) {
        const bool isq = t < NS;
        const int so = ((c * KSTEPS + wave * NS + (isq ? t : t - NS)) * 4) * 1024;
#pragma unroll
        for (int f = 0; f < 4; ++f) r[f] = buf_load16(isq ? rq : rk, vl, so + f * 1024);
    };
    bf16x8 ring[PD][4];
#pragma unroll
    for (int p = 0; p < PD; ++p) load_step(ring[p], 0, p);
    auto advance = [&](bf16x8 (&cur)[4], int c, int cn, int t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) cur[i] = ring[0][i];
#pragma unroll
        for (int p = 0; p + 1 < PD; ++p)
#pragma unroll
            for (int i = 0; i < 4; ++i) ring[p][i] = ring[p + 1][i];
        const int tn = t + PD;
        if (tn < 2 * NS) load_step(ring[PD - 1], c, tn);
        else load_step(ring[PD - 1], cn, tn - 2 * NS);
        __builtin_amdgcn_sched_barrier(0);
    };

    // V tile and w of a chunk: loaded into registers one chunk ahead; stored as V
    // (three buffers: the output rows of chunk c read it during chunk c + 1) and as
    // (w / sigma') (.) V split into bf16 hi + lo (two buffers)
    auto load_v = [&](f32x4 (&rv)[C::NPV], float (&rw)[C::NPV], int c) {
        const size_t t0 = (size_t)c * L;
#pragma unroll
        for (int u = 0; u < C::NPV; ++u) {
            const int idx = min(tid + u * THREADS, C::U_V - 1);
            const int row = idx / (TV / 8), col = min(8 * (idx % (TV / 8)), vcols - 8);
            rv[u] = *reinterpret_cast<const f32x4*>(v + (tinh + t0 + row) * dv + vcol + col);
            rw[u] = ws.w[tokh + t0 + row];
        }
    };
    auto store_v = [&](const f32x4 (&rv)[C::NPV], const float (&rw)[C::NPV], float inv_sig, int c) {
        bf16* vr = sm.v[c % 3];
        bf16* vh = sm.vwh[c & 1];
        bf16* vl2 = sm.vwl[c & 1];
#pragma unroll
        for (int u = 0; u < C::NPV; ++u) {
            const int idx = tid + u * THREADS;
            if ((C::U_V % THREADS == 0) || idx < C::U_V) {
                const int row = idx / (TV / 8), col = 8 * (idx % (TV / 8));
                // columns past d_v hold zeros (their products are never stored)
                const f32x4 val = col < vcols ? rv[u] : f32x4{0, 0, 0, 0};
                *reinterpret_cast<f32x4*>(vr + row * VP + col) = val;
                const bf16x8 vb8 = __builtin_bit_cast(bf16x8, val);
                bf16x8 hh, ll;
                split8w(rw[u] * inv_sig, vb8, hh, ll);
                *reinterpret_cast<bf16x8*>(vh + row * VP + col) = hh;
                *reinterpret_cast<bf16x8*>(vl2 + row * VP + col) = ll;
            }
        }
    };

    // sigma: scale of the registers (C^ = C' / sigma) during a chunk's retrieval;
    // cand, resc, sig_new: the chunk's decay folded in, and whether the registers
    // are rescaled instead (every thread takes the same decision)
    float sigma = 1.0f;
    float cand = ws.alpha[ch0];
    bool resc = cand < SIGMA_MIN;
    float sig_new = resc ? 1.0f : cand;
    {
        f32x4 rv0[C::NPV];
        float rw0[C::NPV];
        load_v(rv0, rw0, 0);
        store_v(rv0, rw0, 1.0f / sig_new, 0);
    }
    f32x4 rv[C::NPV];
    float rw[C::NPV];
    load_v(rv, rw, min(1, nC - 1));
    float alpha_n = ws.alpha[ch0 + min(1, nC - 1)];
    lds_barrier();

    // Output rows of a chunk are finished during the next chunk's retrieval sweep
    // (after its first step), from the partial sums the key parts left in LDS, so
    // that no wave waits for the others between the two sweeps: the one barrier per
    // chunk is at its end.  Operands of the owned blocks, loaded during the chunk:
    f32x4 own[C::NOWN];                 // this wave's own partial retrieval
    bf16x8 pa[C::NOWN][2][2];           // P_loc rows, hi and lo
    f32x4 ga[C::NOWN], gr[C::NOWN], gd[C::NOWN];
    float og[C::NOWN][4];
    float osig = 1.0f;                  // sigma of that chunk's retrieval
    auto load_out = [&](int c) {
        const size_t t0 = (size_t)c * L;
#pragma unroll
        for (int j = 0; j < C::NOWN; ++j) {
            const int b = min(wave + NK * j, NB - 1);
            const int tb = b / CW, x = b % CW;
            // P_loc in operand order: fragment (tb, kk, hi/lo) is 1 KB at ((tb*2+kk)*2+hl) KB
            const char* P = reinterpret_cast<const char*>(ws.P + 2 * (tokh + t0) * L) + lane * 16;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                pa[j][kk][0] = *reinterpret_cast<const bf16x8*>(P + ((tb * 2 + kk) * 2) * 1024);
                pa[j][kk][1] = *reinterpret_cast<const bf16x8*>(P + ((tb * 2 + kk) * 2 + 1) * 1024);
            }
            const size_t tk = tokh + t0 + 16 * tb + 4 * lg;
            ga[j] = *reinterpret_cast<const f32x4*>(ws.a + tk);
            gr[j] = *reinterpret_cast<const f32x4*>(ws.r + tk);
            gd[j] = *reinterpret_cast<const f32x4*>(ws.rden + tk);
            const int col = vcol + min(16 * x, vcols - 16) + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) og[j][i] = o_pre[(tinh + t0 + 16 * tb + 4 * lg + i) * dv + col];
        }
    };
    auto output = [&](int c) {
        const size_t t0 = (size_t)c * L;
        const float* red = sm.red[c & 1];
        const bf16* vr = sm.v[c % 3];
        if (!C::OUT_PREFETCH) load_out(c);
#pragma unroll
        for (int j = 0; j < C::NOWN; ++j) {
            const int b = wave + NK * j;
            if (b >= NB) continue;
            const int tb = b / CW, x = b % CW;
            f32x4 inter = own[j], intra = {0, 0, 0, 0};
#pragma unroll
            for (int p = 0; p < NK - 1; ++p)
                inter += *reinterpret_cast<const f32x4*>(red + (b * (NK - 1) + p) * 256 + lane * 4);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16* vp = vr + (32 * kk + 8 * lg + (ln >> 2)) * VP + 16 * x + 4 * (ln & 3);
                const bf16x8 bop = cat(lds_read_tr(vp), lds_read_tr(vp + 4 * VP));
                intra = mfma(pa[j][kk][0], bop, intra);
                intra = mfma(pa[j][kk][1], bop, intra);
            }
            f32x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float num = gr[j][i] * intra[i] + ga[j][i] * osig * inter[i];
                const float o = __builtin_amdgcn_rcpf(1.0f + __expf(-og[j][i]));
                y[i] = o * num * gd[j][i];
            }
            const f32x4 tq = quad_transpose(y, ln & 3);
            const int col = 16 * x + 4 * (ln >> 2);
            if (col < vcols)
                *reinterpret_cast<bf16x4*>(h + (tinh + t0 + 16 * tb + 4 * lg + (ln & 3)) * dv + vcol + col) =
                    bf16x4{(bf16)tq[0], (bf16)tq[1], (bf16)tq[2], (bf16)tq[3]};
        }
    };

    for (int c = 0; c < nC; ++c) {
        const int cn = min(c + 1, nC - 1);         // chunk whose operands are prefetched at the end

        // --- retrieval sweep: acc = Q C^ over this wave's key rows -------------
        f32x4 acc[LB][CW];
#pragma unroll
        for (int tb = 0; tb < LB; ++tb)
#pragma unroll
            for (int x = 0; x < CW; ++x) acc[tb][x] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            bf16x8 cur[4];
            advance(cur, c, cn, s);
            bf16x8 bhi[CW], blo[CW];
#pragma unroll
            for (int x = 0; x < CW; ++x) split8(st[x][2 * s], st[x][2 * s + 1], bhi[x], blo[x]);
#pragma unroll
            for (int tb = 0; tb < LB; ++tb)
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    acc[tb][x] = mfma(cur[tb], bhi[x], acc[tb][x]);
                    acc[tb][x] = mfma(cur[tb], blo[x], acc[tb][x]);
                }
            if (s == 0 && c > 0) output(c - 1);
        }
        osig = sigma;
        if (C::OUT_PREFETCH) load_out(c);
        // partial sums of the blocks other waves own (owner of block b: wave b % NK);
        // the owner keeps its own
        {
            float* red = sm.red[c & 1];
#pragma unroll
            for (int tb = 0; tb < LB; ++tb)
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    const int b = tb * CW + x, owner = b % NK;
                    if (owner != wave) {
                        const int slot = wave < owner ? wave : wave - 1;
                        *reinterpret_cast<f32x4*>(red + (b * (NK - 1) + slot) * 256 + lane * 4) = acc[tb][x];
                    } else {
                        own[b / NK] = acc[tb][x];
                    }
                }
        }

        // --- update sweep: C^ += K^T ((w / sigma') V)_{hi+lo} -------------------
        if (resc) {
#pragma unroll
            for (int x = 0; x < CW; ++x)
#pragma unroll
                for (int b = 0; b < 2 * NS; ++b) st[x][b] *= cand;
        }
        {
            bf16x8 vwh[CW][2], vwl[CW][2];
            const bf16* vh = sm.vwh[c & 1];
            const bf16* vl2 = sm.vwl[c & 1];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int x = 0; x < CW; ++x) {
                    const int off = (32 * kk + 8 * lg + (ln >> 2)) * VP + 16 * x + 4 * (ln & 3);
                    vwh[x][kk] = cat(lds_read_tr(vh + off), lds_read_tr(vh + off + 4 * VP));
                    vwl[x][kk] = cat(lds_read_tr(vl2 + off), lds_read_tr(vl2 + off + 4 * VP));
                }
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 cur[4];
                advance(cur, c, cn, NS + s);
#pragma unroll
                for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int x = 0; x < CW; ++x) {
                            st[x][2 * s + jt] = mfma(cur[2 * jt + kk], vwh[x][kk], st[x][2 * s + jt]);
                            st[x][2 * s + jt] = mfma(cur[2 * jt + kk], vwl[x][kk], st[x][2 * s + jt]);
                        }
            }
        }
        sigma = sig_new;
        // the next chunk's tiles: (w / sigma') (.) V into the half chunk c - 1's update
        // read, V into the buffer chunk c - 2's output rows read (both before the last
        // barrier).  (After the last chunk this rewrites buffers nobody reads.)
        cand = sigma * alpha_n;
        resc = cand < SIGMA_MIN;
        sig_new = resc ? 1.0f : cand;
        store_v(rv, rw, 1.0f / sig_new, c + 1);
        load_v(rv, rw, min(c + 2, nC - 1));
        alpha_n = ws.alpha[ch0 + min(c + 2, nC - 1)];
        // every wave's partial sums and the next chunk's tiles are in LDS before any
        // wave reads them; the sums of chunk c - 1 (read during this chunk) are
        // overwritten only after the next barrier
        lds_barrier();
    }
    output(nC - 1);

    if (seg != G - 1) return;
#pragma unroll
    for (int x = 0; x < CW; ++x) {
        if (16 * x >= vcols) continue;
#pragma unroll
        for (int b = 0; b < 2 * NS; ++b)
            *reinterpret_cast<f32x4*>(Cout + ((size_t)bh * dv + vcol + 16 * x + ln) * DQ + kw + 32 * (b / 2) + 8 * lg +
                                      4 * (b % 2)) = st[x][b] * sigma;
    }
    if (vt == 0) {
        for (int j = tid; j < DQ; j += THREADS) nout[(size_t)bh * DQ + j] = ws.nfin[(size_t)bh * DQ + j];
        if (tid == 0) mout[bh] = ws.mfin[bh];
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <int L>
hipError_t launch_prep(const FwdArgs& a, const Ws& w) {
    dim3 grid(a.S / L, a.B * a.NH);
    // the streaming scan's operand-ordered copies (64-token chunks only)
    if (L == 64 && w.qs != nullptr)
        hipLaunchKernelGGL((chunk_prep_kernel<L, true>), grid, dim3(PREP_THREADS), 0, a.stream,
                           (const bf16*)a.q, (const bf16*)a.k, a.i_pre, a.f_pre, a.S, a.Sx, a.dqk, w);
    else
        hipLaunchKernelGGL((chunk_prep_kernel<L, false>), grid, dim3(PREP_THREADS), 0, a.stream,
                           (const bf16*)a.q, (const bf16*)a.k, a.i_pre, a.f_pre, a.S, a.Sx, a.dqk, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int heads = a.B * a.NH;
    const int gs_parts = max((a.dqk + GS_COLS - 1) / GS_COLS, min(64, (256 + heads - 1) / heads));
    hipLaunchKernelGGL((gate_scan_kernel<L>), dim3(gs_parts, heads), dim3(GS_THREADS), 0, a.stream,
                       w, a.S, a.dqk, a.n0, a.m0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((den_kernel<L>), dim3(a.S / L, a.B * a.NH), dim3(DEN_THREADS), 0, a.stream,
                       (const bf16*)a.q, w, a.S, a.Sx, a.dqk);
    return hipGetLastError();
}

// Sequence segments per head: enough that (heads x value tiles x segments) covers
// the chip, each segment at least 4 chunks long.  Long sequences over few heads
// (the long-context shape) are otherwise a handful of sequential workgroups.
template <class C>
int segments(const FwdArgs& a) {
    const int units = a.B * a.NH * ((a.dv + C::TV - 1) / C::TV);
    const int nC = a.S / C::L;
    int G = 1;
    if (a.dqk % 64 != 0) return G;            // the segment-state waves cover whole 64-key blocks
    while (2 * G <= SC_MAXG && units * 2 * G <= 256 && nC % (2 * G) == 0 && nC / (2 * G) >= 4) G *= 2;
    return G;
}

template <class C, bool EPI>
hipError_t launch_scan2(const FwdArgs& a, const Ws& w, int G) {
    constexpr int L = C::L;
    const int heads = a.B * a.NH;
    if (G > 1) {
        dim3 sgrid(((a.dqk + SS_TILE - 1) / SS_TILE) * ((a.dv + SS_TILE - 1) / SS_TILE), (G - 1) * w.sp, heads);
        hipLaunchKernelGGL((seg_state_kernel<L>), sgrid, dim3(SS_THREADS), 0, a.stream,
                           (const bf16*)a.k, (const bf16*)a.v, w, a.S, a.Sx, a.dqk, a.dv, G);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t quads = (size_t)a.dv * a.dqk / 4;
        hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)((quads + SC_THREADS - 1) / SC_THREADS), heads),
                           dim3(SC_THREADS), 0, a.stream, w, a.S / L, G, a.dqk, a.dv, a.C0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n_vt = (a.dv + C::TV - 1) / C::TV;
    const int nwg = heads * G * n_vt;
    const int remap = (nwg % 8 == 0) ? 1 : 0;
    const EpiArgs ep = {(const bf16*)a.ep_x, (const bf16*)a.ep_z, a.ep_gw, a.ep_gb, a.ep_sw, a.ep_eps, a.ep_act, a.NH};
    hipLaunchKernelGGL((chunk_scan2_kernel<C, EPI>), dim3(nwg), dim3(C::THREADS), 0, a.stream,
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.o_pre, w, a.S, a.Sx, G, a.dv, n_vt, remap,
                       a.C0, (bf16*)a.h, a.C, a.n, a.m, ep);
    return hipGetLastError();
}

template <class C>
hipError_t launch_scan4(const FwdArgs& a, const Ws& w, int G) {
    constexpr int L = C::L;
    const int heads = a.B * a.NH;
    if (G > 1) {
        dim3 sgrid(((a.dqk + SS_TILE - 1) / SS_TILE) * ((a.dv + SS_TILE - 1) / SS_TILE), (G - 1) * w.sp, heads);
        hipLaunchKernelGGL((seg_state_kernel<L>), sgrid, dim3(SS_THREADS), 0, a.stream,
                           (const bf16*)a.k, (const bf16*)a.v, w, a.S, a.Sx, a.dqk, a.dv, G);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        const size_t quads = (size_t)a.dv * a.dqk / 4;
        hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)((quads + SC_THREADS - 1) / SC_THREADS), heads),
                           dim3(SC_THREADS), 0, a.stream, w, a.S / L, G, a.dqk, a.dv, a.C0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int n_vt = (a.dv + C::TV - 1) / C::TV;
    const int nwg = heads * G * n_vt;
    const int remap = (nwg % 8 == 0) ? 1 : 0;
    hipLaunchKernelGGL((chunk_scan4_kernel<C>), dim3(nwg), dim3(C::THREADS), 0, a.stream,
                       (const bf16*)a.v, a.o_pre, w, a.S, a.Sx, G, a.dv, n_vt, remap,
                       a.C0, (bf16*)a.h, a.C, a.n, a.m);
    return hipGetLastError();
}

typedef hipError_t (*RunFn)(const FwdArgs&, int, size_t*);
RunFn pick_pipelined(int L, int dqk);

template <int DQ, int NK, int CW, int MINB, int PD, bool OP>
hipError_t run4(const FwdArgs& a, int stage, size_t* bytes) {
    using C = Scan4Cfg<DQ, NK, CW, MINB, PD, OP>;
    // the operand copies of one head are addressed with 32-bit buffer offsets
    if ((size_t)a.S * DQ * sizeof(bf16) > (size_t)INT_MAX) return pick_pipelined(C::L, DQ)(a, stage, bytes);
    if (stage == 3) {                     // the streaming form writes h as is
        *bytes = 0;
        return hipSuccess;
    }
    if (stage == 1 && a.ep_x != nullptr) return hipErrorNotSupported;
    const int G = segments<C>(a);
    if (stage == 2) {
        *bytes = ws_bytes((size_t)a.B * a.NH, a.S, C::L, a.dqk, a.dv, G, true);
        return hipSuccess;
    }
    Ws w = ws_layout(a.ws, (size_t)a.B * a.NH, a.S, C::L, a.dqk, a.dv, G, true);
    if (stage == 0) return launch_prep<C::L>(a, w);
    return launch_scan4<C>(a, w, G);
}

// stage 0 = prepare (chunk_prep, gate_scan, den), stage 1 = scan (segments, chunk_scan2),
// stage 2 = workspace size only
// stage 3 = whether this tiling can apply the block epilogue itself (*bytes = 1)
template <int L, int DQ, int NC, int NK, int SB, int MINB, int CW, bool RS>
hipError_t run2(const FwdArgs& a, int stage, size_t* bytes) {
    using C = Scan2Cfg<L, DQ, NC, NK, SB, MINB, CW, RS>;
    // the fused epilogue is built for the 64-column tiles of one wave per SIMD (one key
    // part), with one tile per head: the two-key-part tilings run two waves per SIMD
    // and have no registers left for the epilogue's operands
    constexpr bool EPI_OK = C::TV == 64 && C::NK == 1;
    if (stage == 3) {
        *bytes = (EPI_OK && a.dv <= C::TV) ? 1 : 0;
        return hipSuccess;
    }
    const int G = segments<C>(a);
    if (stage == 2) {
        *bytes = ws_bytes((size_t)a.B * a.NH, a.S, L, a.dqk, a.dv, G, false);
        return hipSuccess;
    }
    Ws w = ws_layout(a.ws, (size_t)a.B * a.NH, a.S, L, a.dqk, a.dv, G, false);
    if (stage == 0) return launch_prep<L>(a, w);
    if (a.ep_x != nullptr) {
        if constexpr (EPI_OK) {
            if (a.dv <= C::TV) return launch_scan2<C, true>(a, w, G);
        }
        return hipErrorNotSupported;
    }
    return launch_scan2<C, false>(a, w, G);
}

// supported (chunk, d_qk) pairs and the tiling used for each:
// (chunk, d_qk, column blocks, key parts, slab, workgroups per CU, column blocks per wave,
//  h stored as 4-column rows after a quad transpose instead of one column per lane)
RunFn pick_pipelined(int L, int dqk) {
#define MLSTM_V2(L_, DQ_, NC_, NK_, SB_, MINB_, CW_, RS_) \
    if (L == L_ && dqk == DQ_) return &run2<L_, DQ_, NC_, NK_, SB_, MINB_, CW_, RS_>;
    // Four waves per workgroup (one per SIMD) let the compiler use the whole
    // register file; eight waves (two per SIMD, key dimension split in two or
    // four parts) hide more latency behind the other wave's MFMAs.  Every entry
    // is chosen by measurement among the tilings that do not spill, except
    // d_qk 1024, whose eight-wave tiling spills a little and still measured
    // fastest (lm 1.3B-class layer shape: 618 us against 660 us for four waves).
    // The transposed row stores save the d_qk 1024 tiling about 7% (its store
    // traffic per slab is the heaviest) and make no measurable difference on the
    // narrower ones.
    MLSTM_V2(32, 128, 4, 1, 128, 1, 1, false)
    MLSTM_V2(32, 384, 3, 1, 128, 1, 1, false)
    MLSTM_V2(64, 64, 4, 1, 64, 1, 1, false)
    MLSTM_V2(64, 128, 4, 1, 128, 1, 1, false)
    MLSTM_V2(64, 192, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 256, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 320, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 384, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 448, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 512, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 576, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 640, 2, 4, 32, 1, 1, true)
    MLSTM_V2(64, 704, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 768, 2, 4, 32, 1, 1, true)
    MLSTM_V2(64, 832, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 896, 2, 4, 32, 1, 1, true)
    MLSTM_V2(64, 960, 4, 2, 32, 1, 1, false)
    MLSTM_V2(64, 1024, 2, 4, 32, 1, 1, true)
#undef MLSTM_V2
    return nullptr;
}

// The streaming scan where it measured faster than the pipelined one: d_qk 1024
// (1.3B-class layer shape: 381 against 481 us for the scan, 468 against 545 us for
// the whole forward) and d_qk 512 (B=4, NH=4, S=2048: 190 against 229 us).  At
// d_qk 640 to 896 its partial-sum exchange and output operands push it past the
// register file (spills), and at d_qk 384 and below it cannot keep two waves per
// SIMD within the LDS, so those stay pipelined.
RunFn pick(int L, int dqk) {
#define MLSTM_V4(DQ_, NK_, CW_, MINB_, PD_, OP_) \
    if (L == 64 && dqk == DQ_) return &run4<DQ_, NK_, CW_, MINB_, PD_, OP_>;
    // (d_qk, key parts = waves, 16-column blocks per wave, workgroups per CU,
    //  operand steps in flight, output operands loaded a chunk ahead)
    MLSTM_V4(1024, 8, 2, 1, 2, true)
    MLSTM_V4(512, 8, 2, 1, 2, true)
#undef MLSTM_V4
    return pick_pipelined(L, dqk);
}

// The chunk size only sets how the recurrence is re-associated: every chunk size
// gives the same result up to rounding.  A 128-token chunk is computed as two
// consecutive 64-token chunks, whose tiles fit the LDS and register budget; a
// 16- or 32-token chunk for a width with no tiling at that chunk is computed in
// 64-token chunks.
int mfma_chunk(const FwdArgs& a) {
    if (a.chunk == 128) return 64;
    if (pick(a.chunk, a.dqk) != nullptr) return a.chunk;
    return 64;
}

}  // namespace

int mfma_fwd_chunk(const FwdArgs& a) {
    if (a.dtype != MLSTM_BF16) return 0;
    const int L = mfma_chunk(a);
    return pick(L, a.dqk) != nullptr ? L : 0;
}

bool mfma_fwd_supported(const FwdArgs& a) {
    const int L = mfma_fwd_chunk(a);
    return L > 0 && a.S % L == 0;
}

size_t mfma_fwd_workspace_bytes(const FwdArgs& a) {
    RunFn f = pick(mfma_chunk(a), a.dqk);
    size_t bytes = 0;
    if (f) (void)f(a, 2, &bytes);
    return bytes;
}

bool mfma_fwd_block_fusable(const FwdArgs& a) {
    if (!mfma_fwd_supported(a)) return false;
    RunFn f = pick(mfma_chunk(a), a.dqk);
    size_t ok = 0;
    if (!f || f(a, 3, &ok) != hipSuccess) return false;
    return ok != 0;
}

hipError_t launch_fwd_mfma_prepare(const FwdArgs& a) {
    RunFn f = pick(mfma_chunk(a), a.dqk);
    if (!f) return hipErrorNotSupported;
    return f(a, 0, nullptr);
}

hipError_t launch_fwd_mfma_scan(const FwdArgs& a) {
    RunFn f = pick(mfma_chunk(a), a.dqk);
    if (!f) return hipErrorNotSupported;
    return f(a, 1, nullptr);
}

}  // namespace mlstm
