// Backward of the mLSTM cell: gradients of the forward from the zero state with
// respect to q, k, v and the three gate pre-activations, given dh.
//
// "xLSTM: Extended Long Short-Term Memory", section 2.3 (the recurrence and its
// parallel form) and section 2.2 (the stabilizer leaves h unchanged, so no
// gradient flows through it).  Per head, with F_t = sum_{j<=t} log sigmoid(f~_j)
// and the stabilizer m_t of the forward,
//   D'_ts = exp(F_t - F_s + i~_s - m_t) <= 1      (s <= t),   S_ts = q_t . k_s
//   num'_t = sum_s D'_ts S_ts v_s,  den'_t = sum_s D'_ts S_ts,
//   N'_t = max(|den'_t|, exp(-m_t)),  u_t = num'_t / N'_t,  h_t = sigmoid(o~_t) (.) u_t
// (num', den', N' are the unstabilized ones times exp(-m_t), a factor that cancels
// in u).  The chain rule in the same stabilized quantities:
//   do~_t  = dh_t (.) u_t (.) g_t (1 - g_t),         du_t = dh_t (.) g_t
//   dnum'_t = du_t / N'_t,   dden'_t = -sign(den'_t) (du_t . u_t) / N'_t  (0 on the floor)
//   dA_ts  = dnum'_t . v_s + dden'_t,   G_ts = dA_ts D'_ts
//   dq_t = sum_s G_ts k_s,   dk_s = sum_t G_ts q_t,   dv_s = sum_t D'_ts S_ts dnum'_t
//   di~_j = k_j . dk_j,   dF_j = q_j . dq_j - k_j . dk_j,
//   df~_j = sigmoid(-f~_j) sum_{t>=j} dF_t
// (the last line collects dlog D_ts = G_ts S_ts over the query and key positions).
//
// Tiled passes over 64-token blocks with fp32 accumulation and fp64 exponent
// arguments (on the vector ALUs here; bf16 inputs with d_qk, d_v <= 512 take the
// MFMA form of the two middle passes further down):
//   bwd_gate_local/fix  per head: F and m (prefix sum, prefix max), fp64, by segments
//   bwd_rows_kernel   per (query block, head): num', den' over key blocks <= it, then
//                     dnum', dden', do~; then dq over the same key blocks
//   bwd_cols_kernel   per (key block, head): dk, dv over query blocks >= it
//   bwd_gates_kernel/fix  per head: di~, df~ (reverse prefix sum), by segments
// From 1024 tokens on, the MFMA form restricts the middle passes to superchunks
// of 256 tokens and reaches the earlier (later) ones through the stabilized state
// (its gradient) at each superchunk boundary: bwd_state_local and bwd_state_scan
// form those states, see the two-level section below.
#include "mlstm_internal.h"

#include <type_traits>
#include <utility>

namespace mlstm {
namespace {

constexpr int BT = 64;           // tokens per block (rows and columns of a score tile)
constexpr int BK = 32;           // contraction slab
constexpr int BW_THREADS = 256;  // 16 x 16 threads, each a 4 x 4 piece of a 64 x 64 tile

struct BwdWs {
    double* F;      // [heads][S] cumulative log forget gate
    double* m;      // [heads][S] stabilizer
    float* dnum;    // [heads][S][dv] num' while it accumulates, then dnum' (vector-ALU path);
                    // the MFMA path keeps dnum' there as bf16 hi [heads][S][dv], then lo
    float* dden;    // [heads][S] dden'
    float* qdq;     // [heads][S] q_t . dq_t (MFMA path)
    double* seg;    // [heads][segments][2] per-segment totals of the two gate scans
    double* gk;     // [heads][S] F_s - i~_s (the key side of the decay's exponent)
    double* rt;     // [heads][S] F_t - m_t (its query side)
};

constexpr int GSEG = 1024;       // tokens per segment of the gate scans

// States of the two-level form (MFMA path, long sequences): see bwd_state_local
struct SuperStates {
    int LS;          // tokens per superchunk (multiple of 64)
    int G;           // superchunks per head; states exist for g = 0 .. G - 2
    bf16* C;         // [heads][G-1][2][d_v][d_qk]: bf16 hi, then lo
    float* n;        // [heads][G-1][d_qk]
    bf16* dC;        // gradients of the states, same layout
    float* dn;       // [heads][G-1][d_qk]
    float* part;     // per-superchunk sums, fp32 [heads][G-1][d_v d_qk + d_qk]
};

// Buffers of the GEMM form (feature widths above 384): see its section below
struct GemmWs {
    int Sp;                  // S rounded up to 128 (the GEMM tile)
    bf16* P;                 // [heads][Sp][Sp] decayed scores, bf16 hi, then lo (same layout)
    bf16* G;                 // [heads][Sp][Sp] score gradients, hi then lo
    float* num;              // [heads][S][d_v] num'
    float* rowpart;          // [heads][S][2 Sp / 128] partial row sums of P
};

int mfma_bwd_width(const BwdArgs& a);

// The GEMM form applies to bf16 with a feature width above 384 and sequences up to
// 16384 tokens (its score-shaped matrices take 8 S_p^2 bytes per head).  Above 512
// the fused tiles do not fit; at 512 it measured 0.80 ms against 1.27 ms for them
// (B=4, NH=4, S=2048), at 384 and below the fused forms are faster.
inline bool bwd_gemm_path(const BwdArgs& a) {
    return a.dtype == MLSTM_BF16 && (a.dqk > 384 || a.dv > 384) && a.S <= 16384 && (long long)a.B * a.NH <= 65535;
}

// Superchunk length of the two-level form: the quadratic tiles shrink to a band of
// LS tokens, at the price of the state products of every 64-token block (about
// three blocks' worth of band work), the per-superchunk state sums and the scans
// over superchunks.  256 measured best from 1024 tokens on (128, 512 and 1024 were
// up to 40% slower); shorter sequences stay one superchunk (G = 1).
inline int bwd_superchunk(const BwdArgs& a) {
    const int S64 = (a.S + 63) / 64 * 64;
    const int LS = 256;
    // workgroups of the per-superchunk kernel and threads of the scan fit a 1-D grid
    const long long heads = (long long)a.B * a.NH;
    const long long local = heads * ((a.dv + 127) / 128) * ((a.dqk + 127) / 128) * ((a.S + LS - 1) / LS);
    const long long scan = heads * (((long long)a.dv * a.dqk + a.dqk) / 4);
    if (mfma_bwd_width(a) == 0 || a.S < 1024 || local > 0x7fffffffLL || scan > 0x7fffffffLL) return S64;
    return LS;
}

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bwd_ws_walk(char* base, const BwdArgs& a, BwdWs* out, SuperStates* ss, GemmWs* gw) {
    const size_t heads = (size_t)a.B * a.NH, S = a.S;
    size_t off = 0;
    auto take = [&](size_t bytes) { char* p = base + off; off += a256(bytes); return p; };
    BwdWs w;
    w.F = (double*)take(heads * S * sizeof(double));
    w.m = (double*)take(heads * S * sizeof(double));
    w.dnum = (float*)take(heads * S * a.dv * sizeof(float));
    w.dden = (float*)take(heads * S * sizeof(float));
    w.qdq = (float*)take(heads * S * sizeof(float));
    w.seg = (double*)take(heads * ((S + GSEG - 1) / GSEG) * 2 * sizeof(double));
    w.gk = (double*)take(heads * S * sizeof(double));
    w.rt = (double*)take(heads * S * sizeof(double));
    SuperStates st;
    st.LS = bwd_superchunk(a);
    st.G = (a.S + st.LS - 1) / st.LS;
    const size_t ns = heads * (size_t)(st.G - 1);
    st.C = (bf16*)take(ns * 2 * a.dv * a.dqk * sizeof(bf16));
    st.dC = (bf16*)take(ns * 2 * a.dv * a.dqk * sizeof(bf16));
    st.n = (float*)take(ns * a.dqk * sizeof(float));
    st.dn = (float*)take(ns * a.dqk * sizeof(float));
    st.part = (float*)take(ns * ((size_t)a.dv * a.dqk + a.dqk) * sizeof(float));
    GemmWs gm = {};
    if (bwd_gemm_path(a)) {
        const size_t Sp = (S + 127) / 128 * 128;
        gm.Sp = (int)Sp;
        gm.P = (bf16*)take(2 * heads * Sp * Sp * sizeof(bf16));
        gm.G = (bf16*)take(2 * heads * Sp * Sp * sizeof(bf16));
        gm.num = (float*)take(heads * S * a.dv * sizeof(float));
        gm.rowpart = (float*)take(heads * S * (2 * Sp / 128) * sizeof(float));
    }
    if (out) *out = w;
    if (ss) *ss = st;
    if (gw) *gw = gm;
    return off;
}

// ---- kernel 1: F and m per head --------------------------------------------
// m_t = max(log f_t + m_{t-1}, i~_t) from m = 0 unrolls to F_t + max(0, max_{s<=t}(i~_s - F_s)).
// Both are prefix scans; they run over segments of GSEG tokens in parallel
// (bwd_gate_local: sums and maxima within the segment, and the segment's totals),
// then bwd_gate_fix adds what the earlier segments carry in.  fp64 throughout.
__global__ __launch_bounds__(BW_THREADS) void bwd_gate_local(const float* __restrict__ i_pre,
                                                             const float* __restrict__ f_pre, int S, BwdWs ws)
{
    __shared__ double part[BW_THREADS / 64];
    const int nseg = (S + GSEG - 1) / GSEG;
    const int sg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = (size_t)bh * S;
    const int ta = sg * GSEG, tb = min(S, ta + GSEG);
    double carry_sum = 0.0, carry_max = -INFINITY;
    for (int t0 = ta; t0 < tb; t0 += BW_THREADS) {
        const int t = t0 + tid;
        double x = t < tb ? log_sigmoid_f64((double)f_pre[base + t]) : 0.0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) part[wave] = x;
        __syncthreads();
        double pre = carry_sum;
        for (int w2 = 0; w2 < wave; ++w2) pre += part[w2];
        const double F = pre + x;                       // within the segment
        double tot = carry_sum;
        for (int w2 = 0; w2 < BW_THREADS / 64; ++w2) tot += part[w2];
        __syncthreads();
        double z = t < tb ? (double)i_pre[base + t] - F : -INFINITY;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(z, off, 64);
            if (lane >= off) z = fmax(z, y);
        }
        if (lane == 63) part[wave] = z;
        __syncthreads();
        double pm = carry_max;
        for (int w2 = 0; w2 < wave; ++w2) pm = fmax(pm, part[w2]);
        double tm = carry_max;
        for (int w2 = 0; w2 < BW_THREADS / 64; ++w2) tm = fmax(tm, part[w2]);
        __syncthreads();
        if (t < tb) {
            ws.F[base + t] = F;
            ws.m[base + t] = fmax(pm, z);               // max over the segment's tokens <= t
        }
        carry_sum = tot;
        carry_max = tm;
    }
    if (tid == 0) {
        ws.seg[((size_t)bh * nseg + sg) * 2] = carry_sum;
        ws.seg[((size_t)bh * nseg + sg) * 2 + 1] = carry_max;
    }
}

__global__ __launch_bounds__(BW_THREADS) void bwd_gate_fix(const float* __restrict__ i_pre, int S, BwdWs ws)
{
    __shared__ double cin[2];
    const int nseg = (S + GSEG - 1) / GSEG;
    const int sg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const size_t base = (size_t)bh * S;
    if (threadIdx.x == 0) {
        // F at the segment's start and max(0, max over earlier tokens of i~ - F)
        double sum = 0.0, mx = 0.0;
        for (int b = 0; b < sg; ++b) {
            const double* p = ws.seg + ((size_t)bh * nseg + b) * 2;
            mx = fmax(mx, p[1] - sum);
            sum += p[0];
        }
        cin[0] = sum;
        cin[1] = mx;
    }
    __syncthreads();
    const double sum = cin[0], mx = cin[1];
    const int ta = sg * GSEG, tb = min(S, ta + GSEG);
    for (int t = ta + threadIdx.x; t < tb; t += BW_THREADS) {
        const double F = sum + ws.F[base + t];
        const double m = F + fmax(mx, ws.m[base + t] - sum);
        ws.F[base + t] = F;
        ws.m[base + t] = m;
        ws.gk[base + t] = F - (double)i_pre[base + t];
        ws.rt[base + t] = F - m;
    }
}

// ---- 64 x 64 tile products on the vector ALUs ---------------------------------
// acc[i][j] += sum_k A(16*ty... ) : thread (ty, tx) owns rows 4ty..4ty+3, cols 4tx..4tx+3.
struct TileSmem {
    float a[BK][BT + 4];     // A slab, k-major
    float b[BK][BT + 4];     // B slab, k-major
};

// acc += A[64 x K] B[K x 64]; a_at(r, k) and b_at(k, c) return 0 outside the data
template <class FA, class FB>
__device__ __forceinline__ void tile_mm(float (&acc)[4][4], int K, TileSmem& sm, FA a_at, FB b_at) {
    const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    for (int k0 = 0; k0 < K; k0 += BK) {
        for (int e = tid; e < BT * BK; e += BW_THREADS) {
            const int r = e / BK, kk = e % BK;
            sm.a[kk][r] = a_at(r, k0 + kk);
            const int kk2 = e / BT, c = e % BT;
            sm.b[kk2][c] = b_at(k0 + kk2, c);
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < BK; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) { av[i] = sm.a[kk][4 * ty + i]; bv[i] = sm.b[kk][4 * tx + i]; }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] += av[i] * bv[j];
        }
        __syncthreads();
    }
}

struct BwdSmem {
    TileSmem t;
    float P[BT][BT + 1];     // a score-sized tile kept for a second product
    double Fr[BT], mr[BT], Fc[BT];
    float ic[BT], dd[BT];
};

template <typename T>
struct BwdIn {
    const T* q; const T* k; const T* v; const T* dh;
    const float* i_pre; const float* f_pre; const float* o_pre;
    int S, dqk, dv;
    int heads, nb;          // heads and 64-token blocks per head
    int LS, G;              // two-level form: tokens per superchunk and superchunks (G = 1: none)
};

// (head, block) of a workgroup of the 1-D grid over blocks x heads: all heads' block
// 0 first, then block 1, ...; block 0 is each kernel's heaviest, so the longest
// workgroups start first and the short ones fill in at the end
__device__ __forceinline__ void grid_block(int heads, int& bh, int& blk) {
    bh = blockIdx.x % heads;
    blk = blockIdx.x / heads;
}

// D'_ts for row t (query) and column s (key) of the current tile pair, 0 above the diagonal
__device__ __forceinline__ float decay(const BwdSmem& sm, int tq, int sk, int r, int c) {
    if (sk > tq) return 0.0f;
    return exp_arg(sm.Fr[r] - sm.Fc[c] + (double)sm.ic[c] - sm.mr[r]);
}

// scores S = Q_rows K_cols^T of a tile pair, into acc
template <typename T>
__device__ __forceinline__ void scores(float (&acc)[4][4], BwdSmem& sm, const BwdIn<T>& in, size_t tokh,
                                       int r0, int c0) {
    const int S = in.S, dqk = in.dqk;
    tile_mm(acc, dqk, sm.t,
            [&](int r, int j) { return (r0 + r < S && j < dqk) ? to_f32(in.q[(tokh + r0 + r) * dqk + j]) : 0.0f; },
            [&](int j, int c) { return (c0 + c < S && j < dqk) ? to_f32(in.k[(tokh + c0 + c) * dqk + j]) : 0.0f; });
}

// dA = dnum'_rows V_cols^T + dden'_rows, into acc (before the dden' term)
template <typename T>
__device__ __forceinline__ void dscores(float (&acc)[4][4], BwdSmem& sm, const BwdIn<T>& in, const BwdWs& ws,
                                        size_t tokh, int r0, int c0) {
    const int S = in.S, dv = in.dv;
    tile_mm(acc, dv, sm.t,
            [&](int r, int j) { return (r0 + r < S && j < dv) ? ws.dnum[(tokh + r0 + r) * dv + j] : 0.0f; },
            [&](int j, int c) { return (c0 + c < S && j < dv) ? to_f32(in.v[(tokh + c0 + c) * dv + j]) : 0.0f; });
}

__device__ __forceinline__ void zero(float (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
}

// ---- kernel 2: per query block -------------------------------------------------
template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_rows_kernel(BwdIn<T> in, BwdWs ws, float* __restrict__ dq,
                                                              float* __restrict__ dout)
{
    __shared__ BwdSmem sm;
    // heavy row blocks (the last ones, with the most key blocks) start first
    const int rb = gridDim.y - 1 - blockIdx.y, bh = blockIdx.x, tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int r0 = rb * BT;
    if (tid < BT) {
        const int t = min(r0 + tid, S - 1);
        sm.Fr[tid] = ws.F[tokh + t];
        sm.mr[tid] = ws.m[tokh + t];
    }
    // clear this block's accumulators (num' in dnum, den' in dden, dq)
    for (int e = tid; e < BT * dv; e += BW_THREADS) {
        const int r = e / dv;
        if (r0 + r < S) ws.dnum[(tokh + r0) * dv + e] = 0.0f;
    }
    for (int e = tid; e < BT * dqk; e += BW_THREADS) {
        const int r = e / dqk;
        if (r0 + r < S) dq[(tokh + r0) * dqk + e] = 0.0f;
    }
    if (tid < BT) sm.dd[tid] = 0.0f;
    __syncthreads();

    // pass 1: num' and den' over the key blocks at or before this one
    for (int cb = 0; cb <= rb; ++cb) {
        const int c0 = cb * BT;
        if (tid < BT) {
            const int s = min(c0 + tid, S - 1);
            sm.Fc[tid] = ws.F[tokh + s];
            sm.ic[tid] = in.i_pre[tokh + s];
        }
        __syncthreads();
        float acc[4][4];
        zero(acc);
        scores(acc, sm, in, tokh, r0, c0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * ty + i, c = 4 * tx + j;
                const bool valid = r0 + r < S && c0 + c < S;
                sm.P[r][c] = valid ? acc[i][j] * decay(sm, r0 + r, c0 + c, r, c) : 0.0f;
            }
        __syncthreads();
        if (tid < BT) {
            float sdn = 0.0f;
            for (int c = 0; c < BT; ++c) sdn += sm.P[tid][c];
            sm.dd[tid] += sdn;
        }
        // num'[rows, value slab] += P V_cols
        for (int j0 = 0; j0 < dv; j0 += BT) {
            float o[4][4];
            zero(o);
            tile_mm(o, BT, sm.t, [&](int r, int s) { return sm.P[r][s]; },
                    [&](int s, int c) {
                        return (c0 + s < S && j0 + c < dv) ? to_f32(in.v[(tokh + c0 + s) * dv + j0 + c]) : 0.0f;
                    });
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * ty + i, c = j0 + 4 * tx + j;
                    if (r0 + r < S && c < dv) ws.dnum[(tokh + r0 + r) * dv + c] += o[i][j];
                }
        }
        __syncthreads();
    }
    // per row: u, do~, dnum', dden'  (one 64-lane wave per row, rows strided over the waves)
    {
        const int lane = tid & 63, wave = tid >> 6;
        for (int r = wave; r < BT; r += BW_THREADS / 64) {
            if (r0 + r >= S) continue;
            const size_t t = tokh + r0 + r;
            const float den = sm.dd[r];
            const float fl = exp_arg(-sm.mr[r]);
            const float N = fmaxf(fabsf(den), fl);
            const float rN = 1.0f / N;
            float du_u = 0.0f;
            for (int j = lane; j < dv; j += 64) {
                const float num = ws.dnum[t * dv + j];
                const float u = num * rN;
                const float g = 1.0f / (1.0f + expf(-in.o_pre[t * dv + j]));
                const float dhv = to_f32(in.dh[t * dv + j]);
                dout[t * dv + j] = dhv * u * g * (1.0f - g);
                const float du = dhv * g;
                du_u += du * u;
                ws.dnum[t * dv + j] = du * rN;
            }
            du_u = wave_sum(du_u);
            if (lane == 0) ws.dden[t] = fabsf(den) > fl ? -(den > 0.0f ? 1.0f : -1.0f) * du_u * rN : 0.0f;
        }
    }
    __syncthreads();
    if (tid < BT) sm.dd[tid] = r0 + tid < S ? ws.dden[tokh + r0 + tid] : 0.0f;
    __syncthreads();

    // pass 2: dq = sum_s (dnum' . v_s + dden') D'_ts k_s
    for (int cb = 0; cb <= rb; ++cb) {
        const int c0 = cb * BT;
        if (tid < BT) {
            const int s = min(c0 + tid, S - 1);
            sm.Fc[tid] = ws.F[tokh + s];
            sm.ic[tid] = in.i_pre[tokh + s];
        }
        __syncthreads();
        float acc[4][4];
        zero(acc);
        dscores(acc, sm, in, ws, tokh, r0, c0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * ty + i, c = 4 * tx + j;
                const bool valid = r0 + r < S && c0 + c < S;
                sm.P[r][c] = valid ? (acc[i][j] + sm.dd[r]) * decay(sm, r0 + r, c0 + c, r, c) : 0.0f;
            }
        __syncthreads();
        for (int j0 = 0; j0 < dqk; j0 += BT) {
            float o[4][4];
            zero(o);
            tile_mm(o, BT, sm.t, [&](int r, int s) { return sm.P[r][s]; },
                    [&](int s, int c) {
                        return (c0 + s < S && j0 + c < dqk) ? to_f32(in.k[(tokh + c0 + s) * dqk + j0 + c]) : 0.0f;
                    });
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = 4 * ty + i, c = j0 + 4 * tx + j;
                    if (r0 + r < S && c < dqk) dq[(tokh + r0 + r) * dqk + c] += o[i][j];
                }
        }
        __syncthreads();
    }
}

// ---- kernel 3: per key block -----------------------------------------------------
template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_cols_kernel(BwdIn<T> in, BwdWs ws, float* __restrict__ dk,
                                                              float* __restrict__ dvv)
{
    __shared__ BwdSmem sm;
    __shared__ float G[BT][BT + 1];
    // heavy key blocks (the first ones, with the most query blocks) start first
    const int cb = blockIdx.y, bh = blockIdx.x, tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int c0 = cb * BT;
    const int nb = (S + BT - 1) / BT;
    if (tid < BT) {
        const int s = min(c0 + tid, S - 1);
        sm.Fc[tid] = ws.F[tokh + s];
        sm.ic[tid] = in.i_pre[tokh + s];
    }
    for (int e = tid; e < BT * dqk; e += BW_THREADS) {
        const int c = e / dqk;
        if (c0 + c < S) dk[(tokh + c0) * dqk + e] = 0.0f;
    }
    for (int e = tid; e < BT * dv; e += BW_THREADS) {
        const int c = e / dv;
        if (c0 + c < S) dvv[(tokh + c0) * dv + e] = 0.0f;
    }
    __syncthreads();
    for (int rb = cb; rb < nb; ++rb) {
        const int r0 = rb * BT;
        if (tid < BT) {
            const int t = min(r0 + tid, S - 1);
            sm.Fr[tid] = ws.F[tokh + t];
            sm.mr[tid] = ws.m[tokh + t];
            sm.dd[tid] = r0 + tid < S ? ws.dden[tokh + r0 + tid] : 0.0f;
        }
        __syncthreads();
        // P = D' (.) S and G = D' (.) dA, both [query rows x key cols]
        float s_acc[4][4], a_acc[4][4];
        zero(s_acc);
        scores(s_acc, sm, in, tokh, r0, c0);
        zero(a_acc);
        dscores(a_acc, sm, in, ws, tokh, r0, c0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 4 * ty + i, c = 4 * tx + j;
                const bool valid = r0 + r < S && c0 + c < S;
                const float d = valid ? decay(sm, r0 + r, c0 + c, r, c) : 0.0f;
                sm.P[r][c] = s_acc[i][j] * d;
                G[r][c] = (a_acc[i][j] + sm.dd[r]) * d;
            }
        __syncthreads();
        // dk[key rows, slab] += G^T Q_rows ;  dv[key rows, slab] += P^T dnum'_rows
        for (int j0 = 0; j0 < dqk; j0 += BT) {
            float o[4][4];
            zero(o);
            tile_mm(o, BT, sm.t, [&](int c, int r) { return G[r][c]; },
                    [&](int r, int j) {
                        return (r0 + r < S && j0 + j < dqk) ? to_f32(in.q[(tokh + r0 + r) * dqk + j0 + j]) : 0.0f;
                    });
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * ty + i, jj = j0 + 4 * tx + j;
                    if (c0 + c < S && jj < dqk) dk[(tokh + c0 + c) * dqk + jj] += o[i][j];
                }
        }
        for (int j0 = 0; j0 < dv; j0 += BT) {
            float o[4][4];
            zero(o);
            tile_mm(o, BT, sm.t, [&](int c, int r) { return sm.P[r][c]; },
                    [&](int r, int j) {
                        return (r0 + r < S && j0 + j < dv) ? ws.dnum[(tokh + r0 + r) * dv + j0 + j] : 0.0f;
                    });
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * ty + i, jj = j0 + 4 * tx + j;
                    if (c0 + c < S && jj < dv) dvv[(tokh + c0 + c) * dv + jj] += o[i][j];
                }
        }
        __syncthreads();
    }
}

// ---- kernel 4: gate gradients per head ----------------------------------------
// di~_j = k_j . dk_j ;  dF_j = q_j . dq_j - k_j . dk_j ;  df~_j = sigmoid(-f~_j) sum_{t>=j} dF_t,
// with q . dq in ws.qdq and k . dk already in di (formed by the column pass of the
// MFMA form, or by bwd_dots_kernel).
// The reverse prefix sum runs over segments of GSEG tokens in parallel: the
// segment's own suffix sums go to ws.F (fp64; F is not needed any more) and its
// total to ws.seg, then bwd_gates_fix adds the later segments' totals.
template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_gates_kernel(BwdIn<T> in, BwdWs ws, const float* __restrict__ di)
{
    __shared__ double part[BW_THREADS / 64];
    const int S = in.S;
    const int nseg = (S + GSEG - 1) / GSEG;
    const int sg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t tokh = (size_t)bh * S;
    const int ta = sg * GSEG, tb = min(S, ta + GSEG);
    double carry = 0.0;
    // walk the segment from its end; within a tile, thread tid holds token end - tid
    for (int e0 = tb - 1; e0 >= ta; e0 -= BW_THREADS) {
        const int t = e0 - tid;
        const double dF = t >= ta ? (double)ws.qdq[tokh + t] - (double)di[tokh + t] : 0.0;
        double x = dF;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) part[wave] = x;
        __syncthreads();
        double pre = carry;
        for (int w2 = 0; w2 < wave; ++w2) pre += part[w2];
        double tot = carry;
        for (int w2 = 0; w2 < BW_THREADS / 64; ++w2) tot += part[w2];
        __syncthreads();
        if (t >= ta) ws.F[tokh + t] = pre + x;
        carry = tot;
    }
    if (tid == 0) ws.seg[((size_t)bh * nseg + sg) * 2] = carry;
}

template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_gates_fix(BwdIn<T> in, BwdWs ws, float* __restrict__ df)
{
    __shared__ double cin;
    const int S = in.S;
    const int nseg = (S + GSEG - 1) / GSEG;
    const int sg = blockIdx.x % nseg, bh = blockIdx.x / nseg;
    const size_t tokh = (size_t)bh * S;
    if (threadIdx.x == 0) {
        double sum = 0.0;                                // later segments, nearest first
        for (int b = sg + 1; b < nseg; ++b) sum += ws.seg[((size_t)bh * nseg + b) * 2];
        cin = sum;
    }
    __syncthreads();
    const int ta = sg * GSEG, tb = min(S, ta + GSEG);
    for (int t = ta + threadIdx.x; t < tb; t += BW_THREADS) {
        const double f = (double)in.f_pre[tokh + t];
        df[tokh + t] = (float)((ws.F[tokh + t] + cin) / (1.0 + exp(f)));    // sigmoid(-f) = 1 / (1 + e^f)
    }
}

// ===========================================================================
// bf16 MFMA form of the two tiled passes (bf16 inputs, max(d_qk, d_v) <= 512)
// ===========================================================================
// Same mathematics as bwd_rows_kernel / bwd_cols_kernel.  A wave owns 16 tokens
// of its block (queries in the row pass, keys in the column pass) and keeps every
// tile with that token index as the MFMA column: score-shaped tiles are held as
// S^T[s][t] (row pass) or S[t][s] (column pass), and per-token vectors as
// X^T[n][t].  In that D layout lane l holds column l%16 and rows 4(l/16) + i, which
// is also a valid B operand when the k-slots 8(l/16) + j are mapped to rows
// {4(l/16) + j} of one 16-row block (j < 4) and of the next (j >= 4); the
// matching A operands are read from LDS either straight (rows contiguous in the
// contraction index) or with the transposing read.
//
// Precision: q, k, v and dh are exact bf16 inputs, but P = S (.) D', G = dA (.) D'
// and dnum' are computed fp32 values.  A single bf16 rounding of them costs up to
// ~1e-1 relative error on the gradients, so each is split into bf16 hi + lo and
// its product taken as two MFMAs (three when both operands are computed: the
// lo x lo term is below fp32 rounding).
constexpr int MB_THREADS = 256;

__device__ __forceinline__ void hilo(float x, bf16& hi, bf16& lo) {
    hi = (bf16)x;
    lo = (bf16)(x - (float)hi);
}

// 16 bytes of bf16 from global memory, or zeros
__device__ __forceinline__ bf16x8 ld8(const bf16* p, bool ok) {
    if (!ok) return bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    return *reinterpret_cast<const bf16x8*>(p);
}

// stage rows [row0, row0 + R) of a [.., d] bf16 tensor into LDS (pitch P), zero
// outside; loads are issued in batches of BATCH per thread before their stores, so
// that many are in flight at once
template <int R, int D, int P, int MAXB>
__device__ __forceinline__ void stage_rows(bf16* dst, const bf16* src, size_t tok0, int row0, int S, int d, int tid) {
    constexpr int U = R * D / 8;                        // 16-byte units
    constexpr int UPT = (U + MB_THREADS - 1) / MB_THREADS;
    constexpr int BATCH = UPT < MAXB ? UPT : MAXB;
#pragma unroll
    for (int b0 = 0; b0 < UPT; b0 += BATCH) {
        bf16x8 tmp[BATCH];
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int u = tid + (b0 + b) * MB_THREADS;
            const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
            tmp[b] = ld8(src + (tok0 + row0 + r) * d + c8, b0 + b < UPT && u < U && row0 + r < S && c8 < d);
        }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
            const int u = tid + (b0 + b) * MB_THREADS;
            const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
            if (b0 + b < UPT && u < U) *reinterpret_cast<bf16x8*>(dst + r * P + c8) = tmp[b];
        }
    }
}

// ===========================================================================
// Two-level form: states at superchunk boundaries (long sequences)
// ===========================================================================
// With superchunks of LS tokens (g = 0, 1, ...; e_g = last token of g, mu_g = m at
// e_g), every key s before superchunk g reaches a query t in g only through the
// stabilized state at the end of superchunk g - 1:
//   C~_g = sum_{s <= e_g} exp(F_{e_g} - F_s + i~_s - mu_g) v_s k_s^T   (n~_g likewise)
//   sum_{s <= e_{g-1}} D'_ts S_ts v_s = beta_t C~_{g-1} q_t,
//   beta_t = exp(F_t - F_{e_{g-1}} + mu_{g-1} - m_t) <= 1.
// So a query needs key blocks of its own superchunk only (the existing tiles,
// restricted to that band) plus beta_t C~_{g-1} q_t; its dq gains
// beta_t (C~_{g-1}^T dnum'_t + n~_{g-1} dden'_t).  In reverse, the gradient of the
// state at the end of superchunk g collects the queries of g + 1 and, decayed, the
// gradient of the next state:
//   dC~_g = sum_{t in g+1} beta_t dnum'_t q_t^T + gamma_{g+1} dC~_{g+1},
//   gamma_{g+1} = exp(F_{e_{g+1}} - F_{e_g} + mu_g - mu_{g+1}) <= 1,
// and a key s of superchunk g gains dv_s += omega_s dC~_g k_s and
// dk_s += omega_s (dC~_g^T v_s + dn~_g), omega_s = exp(F_{e_g} - F_s + i~_s - mu_g).
// Every weight is <= 1 since m is the running max of the log-weights.
constexpr int WK_THREADS = 256;         // the scan
constexpr int LT = 128;                 // local sums: n and j extent of a workgroup's tile
constexpr int LW = LT / 16;             // waves of a local-sum workgroup (one 16-row strip each)
constexpr int LP = LT + 16;             // LDS pitch (bf16) of its token-major tiles (read transposed only:
                                        // 8 banks mod 64 between rows keeps those reads conflict free)

__device__ __forceinline__ size_t state_off(int bh, int g, int G, int dv, int dqk) {
    return ((size_t)bh * (G - 1) + g) * 2 * (size_t)dv * dqk;
}

struct alignas(16) LocalSmem {
    bf16 x[2][64 * LP];      // X tile [token][n] (hi; lo in reverse)
    bf16 y[64 * LP];         // Y tile [token][j]
    float w[64];             // token weights
    float dd[64];            // weights of the vector part
    float vs[4][LT];         // partial sums of the vector
};

// The contribution of one superchunk to one state, for one LT x LT tile of it:
//   forward  L_g = sum_{s in g}     omega_s v_s k_s^T,        l_g = sum omega_s k_s
//   reverse  R_g = sum_{t in g + 1} beta_t dnum'_t q_t^T,     r_g = sum beta_t dden'_t q_t
// (omega and beta relative to the end of superchunk g, as in the states).  One
// workgroup per (tile, state, head) of a 1-D grid, tile fastest; wave w owns rows
// n0 + 16 w .. + 15 of the tile and all its columns.  The next 64 tokens' loads are
// issued before the current tile's products, so memory latency overlaps the MFMAs.
// The sums go to `part` as fp32 [heads][G-1][d_v d_qk + d_qk] (matrix rows n, then
// the vector), and the tiles with n0 == 0 also sum the vector.
template <bool REV>
__global__ __launch_bounds__(64 * LW) void bwd_state_local(BwdIn<bf16> in, BwdWs ws, SuperStates ss,
                                                           float* __restrict__ part)
{
    constexpr int NT = 64 * LW;                     // threads
    constexpr int UPT = 64 * LT / 8 / NT;           // 16-byte units of a tile per thread
    __shared__ LocalSmem sm;
    const int S = in.S, dqk = in.dqk, dv = in.dv, G = ss.G, LS = ss.LS;
    const int tj = (dqk + LT - 1) / LT, tiles = tj * ((dv + LT - 1) / LT);
    const int tile = blockIdx.x % tiles, gh = blockIdx.x / tiles;
    const int g = gh % (G - 1), bh = gh / (G - 1);
    const int n0 = LT * (tile / tj), j0 = LT * (tile % tj);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g4 = lane >> 4;
    const size_t tokh = (size_t)bh * S;
    const bf16* dnh = reinterpret_cast<const bf16*>(ws.dnum);
    const bf16* dnl = dnh + (size_t)in.heads * S * dv;
    const bf16* xs = REV ? dnh : in.v;
    const bf16* ys = REV ? in.q : in.k;
    const bool vec = n0 == 0;
    const int eg = (g + 1) * LS - 1;
    const double Fe = ws.F[tokh + eg], mue = ws.m[tokh + eg];
    const int ta = REV ? (g + 1) * LS : g * LS;
    const int tb = REV ? min(S, (g + 2) * LS) : (g + 1) * LS;

    bf16x8 rx[UPT], rl[UPT], ry[UPT];
    double wa = 0.0, wb = 0.0;              // per-token gate values (tid < 64)
    float wdd = 0.0f;
    bool wok = false;
    auto load = [&](int s0) {
#pragma unroll
        for (int b = 0; b < UPT; ++b) {
            const int u = tid + NT * b, r = u / (LT / 8), c8 = 8 * (u % (LT / 8));
            const int s = s0 + r;
            const bool ok = s < tb;
            const size_t ts = tokh + (ok ? s : ta);
            rx[b] = ld8(xs + ts * dv + n0 + c8, ok && n0 + c8 < dv);
            rl[b] = REV ? ld8(dnl + ts * dv + n0 + c8, ok && n0 + c8 < dv) : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            ry[b] = ld8(ys + ts * dqk + j0 + c8, ok && j0 + c8 < dqk);
        }
        if (tid < 64) {
            const int s = s0 + tid;
            const size_t ts = tokh + (s < tb ? s : ta);
            wa = ws.F[ts];
            wb = REV ? ws.m[ts] : (double)in.i_pre[ts];
            wdd = REV ? ws.dden[ts] : 1.0f;
            wok = s < tb;                    // weight 0 beyond the superchunk
        }
    };

    f32x4 acc[LT / 16];
#pragma unroll
    for (int jb = 0; jb < LT / 16; ++jb) acc[jb] = f32x4{0, 0, 0, 0};
    float vpart[LT / 64];                   // vector partials: column lane + 64 c, tokens = wave (mod 4)
#pragma unroll
    for (int c = 0; c < LT / 64; ++c) vpart[c] = 0.0f;
    load(ta);
    for (int s0 = ta; s0 < tb; s0 += 64) {
        __syncthreads();                     // previous step's tiles consumed
#pragma unroll
        for (int b = 0; b < UPT; ++b) {
            const int u = tid + NT * b, r = u / (LT / 8), c8 = 8 * (u % (LT / 8));
            *reinterpret_cast<bf16x8*>(sm.x[0] + r * LP + c8) = rx[b];
            if (REV) *reinterpret_cast<bf16x8*>(sm.x[1] + r * LP + c8) = rl[b];
            *reinterpret_cast<bf16x8*>(sm.y + r * LP + c8) = ry[b];
        }
        if (tid < 64) {
            // omega_s = exp(F_e - F_s + i~_s - mu_e);  beta_t = exp(F_t - F_e + mu_e - m_t)
            const float wgt = !wok ? 0.0f : REV ? exp_arg(wa - Fe + mue - wb) : exp_arg(Fe - wa + wb - mue);
            sm.w[tid] = wgt;
            sm.dd[tid] = wgt * wdd;
        }
        lds_barrier();
        if (s0 + 64 < tb) load(s0 + 64);     // in flight during the products below
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int trow = 32 * kk + 8 * g4 + (ln >> 2);
            const bf16* xp = sm.x[0] + trow * LP + 16 * wave + 4 * (ln & 3);
            const bf16x8 xv = cat(lds_read_tr(xp), lds_read_tr(xp + 4 * LP));
            bf16x8 xl = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
            if (REV) {
                const bf16* xq = sm.x[1] + trow * LP + 16 * wave + 4 * (ln & 3);
                xl = cat(lds_read_tr(xq), lds_read_tr(xq + 4 * LP));
            }
            const f32x4 w0 = *reinterpret_cast<const f32x4*>(&sm.w[32 * kk + 8 * g4]);
            const f32x4 w1 = *reinterpret_cast<const f32x4*>(&sm.w[32 * kk + 8 * g4 + 4]);
            bf16x8 ah, al;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float xf = (float)xv[e] + (REV ? (float)xl[e] : 0.0f);
                bf16 hi, lo;
                hilo((e < 4 ? w0[e] : w1[e - 4]) * xf, hi, lo);
                ah[e] = hi;
                al[e] = lo;
            }
#pragma unroll
            for (int jb = 0; jb < LT / 16; ++jb) {
                const bf16* yp = sm.y + trow * LP + 16 * jb + 4 * (ln & 3);
                const bf16x8 yv = cat(lds_read_tr(yp), lds_read_tr(yp + 4 * LP));
                acc[jb] = mfma(ah, yv, acc[jb]);
                acc[jb] = mfma(al, yv, acc[jb]);
            }
        }
        if (vec && wave < 4) {
#pragma unroll 4
            for (int r = wave; r < 64; r += 4) {
                const float d = sm.dd[r];
#pragma unroll
                for (int c = 0; c < LT / 64; ++c) vpart[c] += d * (float)sm.y[r * LP + lane + 64 * c];
            }
        }
    }
    // the tile straight from the accumulators: rows n0 + 16 wave + 4 g4 + i, columns
    // j0 + 16 jb + ln (16 consecutive floats per row and instruction)
    const size_t E = (size_t)dv * dqk + dqk;
    float* dst = part + ((size_t)bh * (G - 1) + g) * E;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int n = n0 + 16 * wave + 4 * g4 + i;
        if (n < dv) {
#pragma unroll
            for (int jb = 0; jb < LT / 16; ++jb) {
                const int j = j0 + 16 * jb + ln;
                if (j < dqk) dst[(size_t)n * dqk + j] = acc[jb][i];
            }
        }
    }
    if (vec) {
        if (wave < 4) {
#pragma unroll
            for (int c = 0; c < LT / 64; ++c) sm.vs[wave][lane + 64 * c] = vpart[c];
        }
        __syncthreads();
        if (tid < LT && j0 + tid < dqk)
            dst[(size_t)dv * dqk + j0 + tid] = sm.vs[0][tid] + sm.vs[1][tid] + sm.vs[2][tid] + sm.vs[3][tid];
    }
}

// The states from the per-superchunk sums, element by element in superchunk order:
//   forward  C~_g  = L_g + gamma_g C~_{g-1},     gamma_g = exp(F_{e_g} - F_{e_{g-1}} + mu_{g-1} - mu_g)
//   reverse  dC~_g = R_g + gamma_{g+1} dC~_{g+1}
// (the vectors likewise), stored as bf16 hi + lo (matrices) and fp32 (vectors).
// One thread per 4 consecutive elements of a head's [d_v d_qk + d_qk]; the next
// superchunk's sums are loaded before the current one is finished.
template <bool REV>
__global__ __launch_bounds__(WK_THREADS) void bwd_state_scan(BwdIn<bf16> in, BwdWs ws, SuperStates ss,
                                                             const float* __restrict__ part, long long quads)
{
    const long long qd = (long long)blockIdx.x * WK_THREADS + threadIdx.x;
    if (qd >= quads) return;
    const int dqk = in.dqk, dv = in.dv, G = ss.G, LS = ss.LS;
    const size_t M = (size_t)dv * dqk, E = M + dqk, EQ = E / 4;
    const int bh = (int)(qd / EQ);
    const size_t e = 4 * (size_t)(qd % EQ);
    const size_t tokh = (size_t)bh * in.S;
    const float* src = part + (size_t)bh * (G - 1) * E + e;
    f32x4 c = f32x4{0, 0, 0, 0};
    int g = REV ? G - 2 : 0;
    f32x4 nxt = load4(src + (size_t)g * E);
    for (int step = 0; step < G - 1; ++step, g += REV ? -1 : 1) {
        const f32x4 cur = nxt;
        if (step + 1 < G - 1) nxt = load4(src + (size_t)(REV ? g - 1 : g + 1) * E);
        if (step > 0) {
            const int ec = (g + 1) * LS - 1, ep = REV ? (g + 2) * LS - 1 : g * LS - 1;
            const double Fc = ws.F[tokh + ec], mc = ws.m[tokh + ec];
            const double Fp = ws.F[tokh + ep], mp = ws.m[tokh + ep];
            c *= REV ? exp_arg(Fp - Fc + mc - mp) : exp_arg(Fc - Fp + mp - mc);
        }
        c += cur;
        if (e < M) {
            bf16* hp = (REV ? ss.dC : ss.C) + state_off(bh, g, G, dv, dqk) + e;
            bf16x4 h4, l4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16 hi, lo;
                hilo(c[i], hi, lo);
                h4[i] = hi;
                l4[i] = lo;
            }
            *reinterpret_cast<bf16x4*>(hp) = h4;
            *reinterpret_cast<bf16x4*>(hp + M) = l4;
        } else {
            *reinterpret_cast<f32x4*>((REV ? ss.dn : ss.n) + ((size_t)bh * (G - 1) + g) * dqk + (e - M)) = c;
        }
    }
}

// ---- staging by buffer loads that write LDS directly ----------------------------
// The row and column passes keep one wave per SIMD at the wider tiles, so a load
// round trip through registers leaves the matrix cores idle.  Buffer loads with the
// LDS flag write their 16 bytes per lane straight into LDS (lane l of a wave fills
// bytes 16 l .. 16 l + 15 of a 1 KB run that starts at the LDS address in M0); they
// need no registers, so the next tile's loads are issued before the products on the
// current one and waited for with a partial vmcnt.  They are written as inline
// assembly: the compiler would otherwise order every LDS read after every such load
// still in flight (it does not tell the two LDS buffers apart), which serializes
// exactly the overlap they are for.  Every wait on them is therefore explicit: a
// vmcnt that leaves only younger loads outstanding, then a barrier.
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): a loop whose index
// is a compile-time constant in every copy (register arrays indexed by it stay registers)
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// raw buffer descriptor over [base, base + bytes): loads past the range return zeros
__device__ __forceinline__ u32x4 span_rsrc(const void* base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
    r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
    r[2] = __builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000u;
    return r;
}

// this lane's 16 bytes at byte offset voff of the descriptor's range into LDS at
// byte address la + 16 * lane (la is the wave's, so uniform).  M0 is saved and restored around
// the load (the compiler keeps it as its own); one wait state between the M0 write
// and the load that reads it.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_ptr)p);
}
__device__ __forceinline__ void dma16(unsigned la, unsigned voff, u32x4 rs) {
    unsigned keep;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(keep) : "s"(la), "v"(voff), "s"(rs) : "memory");
}

// wait until at most N of this wave's vector memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// A tile of R rows x D columns in LDS with pitch D + 8 bf16: D / 8 + 1 granules of 16
// bytes per row, the last one padding.  It is filled in LDS order in runs of 1 KB
// (64 granules), dealt to the four waves round robin.
template <int R, int D>
struct DmaTile {
    static constexpr int GR = D / 8 + 1;
    static constexpr int TOT = R * GR;
    static constexpr int NCH = (TOT + 63) / 64;
    static constexpr int MIN_PER_WAVE = NCH / 4;      // loads every wave issues for one tile, at least
};

// The byte offsets of this wave's granules of a tile whose rows are d elements apart,
// one per 1 KB run (c = wave, wave + 4, ...), computed once per kernel: granule u =
// 64 c + lane is row u / GR, column granule u % GR.  Granules past column d and the
// padding granules get an offset beyond any descriptor's range (they land as zeros);
// lanes past the end of the tile get NONE and issue nothing.
template <int R, int D>
struct DmaOffs {
    using T = DmaTile<R, D>;
    static constexpr int NI = (T::NCH + 3) / 4;
    static constexpr unsigned NONE = 0xffffffffu;
    unsigned o[NI];
    __device__ __forceinline__ DmaOffs(int d, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int u = 64 * (wave + 4 * i) + lane;
            const int r = u / T::GR, gc = u - r * T::GR;
            o[i] = u >= T::TOT ? NONE
                   : (gc < D / 8 && 8 * gc < d) ? (unsigned)(r * d + 8 * gc) * 2u : 0x80000000u;
        }
    }
};

// Rows [0, R) of a row-major bf16 block (`rows` rows present, at the stride the
// offsets were made for) into LDS at byte address dst, columns [0, D); rows past `rows` read
// beyond the descriptor's range and land as zeros.
template <int R, int D>
__device__ __forceinline__ void dma_tile(unsigned dst, const bf16* src, int rows, int d, const DmaOffs<R, D>& of,
                                         int wave) {
    using T = DmaTile<R, D>;
    const unsigned bytes = rows > 0 ? (unsigned)(rows < R ? rows : R) * (unsigned)d * 2u : 0u;
    const u32x4 rs = span_rsrc(src, bytes);
#pragma unroll
    for (int i = 0; i < DmaOffs<R, D>::NI; ++i) {
        const int c = wave + 4 * i;
        if (c < T::NCH) {
            if (T::TOT % 64 == 0 || i + 1 < DmaOffs<R, D>::NI) dma16(dst + 1024u * c, of.o[i], rs);
            else if (of.o[i] != DmaOffs<R, D>::NONE) dma16(dst + 1024u * c, of.o[i], rs);
        }
    }
}

// n16 granules (n16 <= 64) of 16 bytes from src into LDS at byte address dst by one
// wave; bytes past `bytes` land as zeros
__device__ __forceinline__ void dma_span(unsigned dst, const void* src, unsigned bytes, int n16, int lane) {
    const u32x4 rs = span_rsrc(src, bytes);
    if (lane < n16) dma16(dst, 16u * lane, rs);
}

// per (head, query block of 64): num', den' over key blocks <= it, then dnum', dden',
// do~ (wave-local), then dq over the same key blocks, and q_t . dq_t.
// Each pass walks a list of tile pairs: first the 64-row slices of the state (two-level
// form), then the key blocks of the band.  The two tiles of a pair go to the two LDS
// buffers; the products on one buffer run while the next pair's tile loads into the
// other (pass 1: K or state hi into sk, then V or state lo into sv; pass 2 the other
// way round, because dA needs V before dq needs K).
template <int D>
__global__ __launch_bounds__(MB_THREADS, D <= 256 ? 2 : 1) void bwd_rows_mfma(BwdIn<bf16> in, BwdWs ws, SuperStates ss,
                                                          float* __restrict__ dq, float* __restrict__ dout)
{
    constexpr int P = D + 8;
    constexpr int NB = D / 16, KS = D / 32;
    // Up to width 256 two workgroups share a CU (two waves per SIMD, 256 registers
    // each): fewer operands are read ahead there.
    constexpr int GB = D <= 256 ? 2 : 4;        // value / key blocks whose operands are read together
    static_assert(NB % GB == 0, "width must be a multiple of 64");
    __shared__ __attribute__((aligned(16))) bf16 sk[64 * P];
    __shared__ __attribute__((aligned(16))) bf16 sv[64 * P];
    __shared__ __attribute__((aligned(16))) double sgs[2][64];   // F_s - i~_s of a key block, by its parity
    int bh, rb;
    grid_block(in.heads, bh, rb);
    rb = in.nb - 1 - rb;                        // the last query blocks have the most key blocks
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int r0 = rb * 64;
    const int t = r0 + 16 * wave + ln;          // this lane's query
    const bool tval = t < S;
    const double Rt = tval ? ws.rt[tokh + t] : 0.0;
    const float fl = tval ? exp_arg(-ws.m[tokh + t]) : 1.0f;
    // two-level form: key blocks of this superchunk only, the earlier ones through the
    // state at the end of the previous superchunk, weighted by beta_t
    const int sg = rb * 64 / in.LS;                 // superchunk of this query block
    const int cb_lo = sg * (in.LS / 64);
    float beta = 0.0f;
    const bf16* Chi = ss.C;
    const bf16* Clo = ss.C;
    int nsl = 0;                                    // state slices of 64 rows
    if (sg > 0) {
        const int ep = sg * in.LS - 1;
        if (tval) beta = exp_arg(Rt - ws.F[tokh + ep] + ws.m[tokh + ep]);
        Chi = ss.C + state_off(bh, sg - 1, in.G, dv, dqk);
        Clo = Chi + (size_t)dv * dqk;
        nsl = (dv + 63) / 64;
    }
    const int np = nsl + rb - cb_lo + 1;            // tile pairs of each pass

    // loads of the tiles of pair p: state rows (hi, lo) or key block rows (K, V); the
    // key block's F_s - i~_s goes with the tile whose products come first
    const DmaOffs<64, D> ofk(dqk, wave, lane), ofv(dv, wave, lane);
    const unsigned ak = lds_addr(sk), av = lds_addr(sv), ag = lds_addr(sgs);
    auto dma_state = [&](unsigned dst, const bf16* base, int p) __attribute__((always_inline)) {
        dma_tile<64, D>(dst, base + (size_t)64 * p * dqk, dv - 64 * p, dqk, ofk, wave);
    };
    auto dma_keys = [&](unsigned dst, const bf16* x, int d, const DmaOffs<64, D>& of, int cb, bool with_gs)
                        __attribute__((always_inline)) {
        dma_tile<64, D>(dst, x + (tokh + 64 * cb) * d, S - 64 * cb, d, of, wave);
        if (with_gs && wave == 1)
            dma_span(ag + 512u * (cb & 1), ws.gk + tokh + 64 * cb, 8u * (unsigned)min(64, S - 64 * cb), 32, lane);
    };
    auto issue1_first = [&](int p) __attribute__((always_inline)) {
        if (p >= np) return;
        if (p < nsl) dma_state(ak, Chi, p);
        else dma_keys(ak, in.k, dqk, ofk, cb_lo + p - nsl, true);
    };
    auto issue1_second = [&](int p) __attribute__((always_inline)) {
        if (p >= np) return;
        if (p < nsl) dma_state(av, Clo, p);
        else dma_keys(av, in.v, dv, ofv, cb_lo + p - nsl, false);
    };
    auto issue2_first = [&](int p) __attribute__((always_inline)) {
        if (p >= np) return;
        if (p < nsl) dma_state(av, Clo, p);
        else dma_keys(av, in.v, dv, ofv, cb_lo + p - nsl, true);
    };
    auto issue2_second = [&](int p) __attribute__((always_inline)) {
        if (p >= np) return;
        if (p < nsl) dma_state(ak, Chi, p);
        else dma_keys(ak, in.k, dqk, ofk, cb_lo + p - nsl, false);
    };
    // One tile is in flight at a time: before the products on a tile, wait for its
    // loads and pass a barrier (after which every wave is done with the other
    // buffer), then issue the other buffer's next tile, which loads during these
    // products.
    auto wait_all = [&]() __attribute__((always_inline)) {
        wait_vm<0>();
        __syncthreads();
    };
    issue1_first(0);

    // q_t as B operands: k-slot 8g + j <-> key dimension 32 kk + 8g + j
    bf16x8 qb[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qb[kk] = ld8(in.q + (tokh + t) * dqk + 32 * kk + 8 * g, tval && 32 * kk + 8 * g < dqk);
    // den'_t starts from beta_t n~ . q_t (lane partials; loaded here, before the pipeline
    // has loads of its own in flight)
    float den = 0.0f;
    if (sg > 0) {
        const float* nt = ss.n + ((size_t)bh * (in.G - 1) + sg - 1) * dqk;
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const int j = 32 * kk + 8 * g;
            if (j < dqk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) den += nt[j + e] * (float)qb[kk][e];
            }
        }
        den *= beta;
    }

    // D'[s][t] for this lane's 16 entries of a tile pair (s = 16 sb + 4g + i)
    auto decay4 = [&](float (&d)[4][4], int c0, const double* gs) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 16 * sb + 4 * g + i;
                d[sb][i] = (tval && c0 + sl <= t) ? exp_arg(Rt - gs[sl]) : 0.0f;
            }
    };

    // ---- pass 1: num'^T[n][t] and den_t -------------------------------------
    f32x4 num[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) num[nb] = f32x4{0, 0, 0, 0};
    // num'^T[n][t] = beta_t (C~ q_t)[n] over the state slices (the state rows take the
    // place of key rows)
    static_for<D / 64>([&](auto slc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        if (sl >= nsl) return;
        wait_all();
        issue1_second(sl);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bf16x8 a[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) a[sb] = *reinterpret_cast<const bf16x8*>(sk + (16 * sb + ln) * P + 32 * kk + 8 * g);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) num[4 * sl + sb] = mfma(a[sb], qb[kk], num[4 * sl + sb]);
        }
        wait_all();
        issue1_first(sl + 1);
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            bf16x8 a[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) a[sb] = *reinterpret_cast<const bf16x8*>(sv + (16 * sb + ln) * P + 32 * kk + 8 * g);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) num[4 * sl + sb] = mfma(a[sb], qb[kk], num[4 * sl + sb]);
        }
    });
    if (sg > 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) num[nb] *= beta;
    }
    for (int cb = cb_lo; cb <= rb; ++cb) {
        const int p = nsl + cb - cb_lo;
        const int c0 = 64 * cb;
        wait_all();
        issue1_second(p);
        f32x4 st[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) st[sb] = f32x4{0, 0, 0, 0};
        constexpr int KB = D <= 256 ? 1 : 2;     // key slabs whose score operands are read together
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += KB) {
            bf16x8 a[KB][4];
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    a[j][sb] = k0 + j < KS ? *reinterpret_cast<const bf16x8*>(sk + (16 * sb + ln) * P + 32 * (k0 + j) + 8 * g)
                                           : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    if (k0 + j < KS) st[sb] = mfma(a[j][sb], qb[k0 + j < KS ? k0 + j : 0], st[sb]);
        }
        float d[4][4];
        decay4(d, c0, sgs[cb & 1]);
        bf16x8 ph[2], pl[2];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = st[sb][i] * d[sb][i];
                den += pv;
                bf16 hi, lo;
                hilo(pv, hi, lo);
                ph[sb >> 1][4 * (sb & 1) + i] = hi;
                pl[sb >> 1][4 * (sb & 1) + i] = lo;
            }
        wait_all();
        issue1_first(p + 1);
        // operands of GB value blocks read together, then their products with
        // consecutive MFMAs on independent accumulators (LDS latency overlaps)
#pragma unroll
        for (int nb0 = 0; nb0 < NB; nb0 += GB) {
            bf16x8 a[GB][2];
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const bf16* vp = sv + (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (nb0 + j) + 4 * (ln & 3);
                    a[j][pr] = cat(lds_read_tr(vp), lds_read_tr(vp + 16 * P));
                }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                for (int j = 0; j < GB; ++j) num[nb0 + j] = mfma(a[j][pr], ph[pr], num[nb0 + j]);
#pragma unroll
                for (int j = 0; j < GB; ++j) num[nb0 + j] = mfma(a[j][pr], pl[pr], num[nb0 + j]);
            }
        }
    }
    // pass 2's first tile loads during the per-query phase, once every wave is done
    // with the last pass-1 tile in its buffer
    __syncthreads();
    issue2_first(0);

    // ---- per query: u, do~, dnum', dden' ------------------------------------
    den += __shfl_xor(den, 16, 64);
    den += __shfl_xor(den, 32, 64);
    const float rN = 1.0f / fmaxf(fabsf(den), fl);
    float duu = 0.0f;
    const bf16* dhp = in.dh + (tokh + t) * dv;
    const float* op = in.o_pre + (tokh + t) * dv;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int n0 = 16 * nb + 4 * g;
        if (tval && n0 < dv) {
            const f32x4 o4 = load4(op + n0), dh4 = load4(dhp + n0);
            f32x4 do4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = num[nb][i] * rN;
                const float gg = sigmoid(o4[i]);
                do4[i] = dh4[i] * u * gg * (1.0f - gg);
                const float du = dh4[i] * gg;
                duu += du * u;
                num[nb][i] = du * rN;
            }
            *reinterpret_cast<f32x4*>(dout + (tokh + t) * dv + n0) = do4;
        } else {
            num[nb] = f32x4{0, 0, 0, 0};
        }
    }
    duu += __shfl_xor(duu, 16, 64);
    duu += __shfl_xor(duu, 32, 64);
    const float dd = (tval && fabsf(den) > fl) ? -(den > 0.0f ? 1.0f : -1.0f) * duu * rN : 0.0f;
    if (tval && g == 0) ws.dden[tokh + t] = dd;
    // dnum' for the column pass (bf16 hi, then lo) and as B operands here
    bf16* dnh_g = reinterpret_cast<bf16*>(ws.dnum);
    bf16* dnl_g = dnh_g + (size_t)in.heads * S * dv;
    bf16x8 dnh[NB / 2], dnl[NB / 2];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        bf16x4 h4, l4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16 hi, lo;
            hilo(num[nb][i], hi, lo);
            h4[i] = hi;
            l4[i] = lo;
            dnh[nb >> 1][4 * (nb & 1) + i] = hi;
            dnl[nb >> 1][4 * (nb & 1) + i] = lo;
        }
        const int n0 = 16 * nb + 4 * g;
        if (tval && n0 < dv) {
            *reinterpret_cast<bf16x4*>(dnh_g + (tokh + t) * dv + n0) = h4;
            *reinterpret_cast<bf16x4*>(dnl_g + (tokh + t) * dv + n0) = l4;
        }
    }

    // ---- pass 2: dq^T[j][t] += K^T G^T, G^T = (V dnum'^T + dden') (.) D' ------
    f32x4 dqa[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) dqa[jb] = f32x4{0, 0, 0, 0};
    // dq^T[j][t] = beta_t (C~^T dnum'_t + n~ dden'_t)[j]: transposing reads of the
    // state slices, whose n order follows dnum''s k-slots (as V's in pass 1); the lo
    // slice (in sv) first, then the hi one (in sk)
    constexpr int GI = D <= 256 ? GB : 2;   // fewer operands in flight at the widest tiles
    static_for<D / 64>([&](auto slc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        if (sl >= nsl) return;
        wait_all();
        issue2_second(sl);
#pragma unroll
        for (int jb0 = 0; jb0 < NB; jb0 += GI) {
            bf16x8 a[GI][2];
#pragma unroll
            for (int j = 0; j < GI; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int off = (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (jb0 + j) + 4 * (ln & 3);
                    a[j][pr] = cat(lds_read_tr(sv + off), lds_read_tr(sv + off + 16 * P));
                }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr)
#pragma unroll
                for (int j = 0; j < GI; ++j) dqa[jb0 + j] = mfma(a[j][pr], dnh[2 * sl + pr], dqa[jb0 + j]);
        }
        wait_all();
        issue2_first(sl + 1);
#pragma unroll
        for (int jb0 = 0; jb0 < NB; jb0 += GI) {
            bf16x8 a[GI][2];
#pragma unroll
            for (int j = 0; j < GI; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int off = (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (jb0 + j) + 4 * (ln & 3);
                    a[j][pr] = cat(lds_read_tr(sk + off), lds_read_tr(sk + off + 16 * P));
                }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                for (int j = 0; j < GI; ++j) dqa[jb0 + j] = mfma(a[j][pr], dnh[2 * sl + pr], dqa[jb0 + j]);
#pragma unroll
                for (int j = 0; j < GI; ++j) dqa[jb0 + j] = mfma(a[j][pr], dnl[2 * sl + pr], dqa[jb0 + j]);
            }
        }
    });
    if (sg > 0) {
#pragma unroll
        for (int jb = 0; jb < NB; ++jb) dqa[jb] *= beta;
    }
    for (int cb = cb_lo; cb <= rb; ++cb) {
        const int p = nsl + cb - cb_lo;
        const int c0 = 64 * cb;
        wait_all();
        issue2_second(p);
        f32x4 da[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) da[sb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int pr = 0; pr < NB / 2; ++pr) {
            bf16x8 a[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const bf16* vp = sv + (16 * sb + ln) * P + 32 * pr + 4 * g;
                a[sb] = cat(*reinterpret_cast<const bf16x4*>(vp), *reinterpret_cast<const bf16x4*>(vp + 16));
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) da[sb] = mfma(a[sb], dnh[pr], da[sb]);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) da[sb] = mfma(a[sb], dnl[pr], da[sb]);
        }
        float d[4][4];
        decay4(d, c0, sgs[cb & 1]);
        bf16x8 gh[2], gl[2];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bf16 hi, lo;
                hilo((da[sb][i] + dd) * d[sb][i], hi, lo);
                gh[sb >> 1][4 * (sb & 1) + i] = hi;
                gl[sb >> 1][4 * (sb & 1) + i] = lo;
            }
        wait_all();
        issue2_first(p + 1);
#pragma unroll
        for (int jb0 = 0; jb0 < NB; jb0 += GB) {
            bf16x8 a[GB][2];
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const bf16* kp = sk + (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (jb0 + j) + 4 * (ln & 3);
                    a[j][pr] = cat(lds_read_tr(kp), lds_read_tr(kp + 16 * P));
                }
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                for (int j = 0; j < GB; ++j) dqa[jb0 + j] = mfma(a[j][pr], gh[pr], dqa[jb0 + j]);
#pragma unroll
                for (int j = 0; j < GB; ++j) dqa[jb0 + j] = mfma(a[j][pr], gl[pr], dqa[jb0 + j]);
            }
        }
    }
    // the state's share beta_t n~ dden'_t, loaded now that no tile loads are in flight
    const float bdd = beta * dd;
    const float* nt = ss.n + ((size_t)bh * (in.G - 1) + (sg > 0 ? sg - 1 : 0)) * dqk;
    float qdq = 0.0f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
        const int j0 = 16 * jb + 4 * g;
        if (tval && j0 < dqk) {
            if (sg > 0) dqa[jb] += bdd * load4(nt + j0);
            *reinterpret_cast<f32x4*>(dq + (tokh + t) * dqk + j0) = dqa[jb];
            const f32x4 q4 = load4(in.q + (tokh + t) * dqk + j0);
#pragma unroll
            for (int i = 0; i < 4; ++i) qdq += q4[i] * dqa[jb][i];
        }
    }
    qdq += __shfl_xor(qdq, 16, 64);
    qdq += __shfl_xor(qdq, 32, 64);
    if (tval && g == 0) ws.qdq[tokh + t] = qdq;
}

// per (head, key block of 64): dk, dv over query blocks >= it (QB queries at a
// time), and k_s . dk_s (= di~_s).  Items: first the QB-row slices of the state
// gradient (two-level form; hi and lo), then the query slabs of the band (Q, dnum' hi,
// dnum' lo and the slab's F_t - m_t and dden'_t).  With two LDS sets (all widths up to
// 384) the next item loads into one set while the products run on the other.
template <int D, int QB>
__global__ __launch_bounds__(MB_THREADS) void bwd_cols_mfma(BwdIn<bf16> in, BwdWs ws, SuperStates ss,
                                                          float* __restrict__ dk,
                                                          float* __restrict__ dvv, float* __restrict__ di)
{
    constexpr int P = D + 8;
    constexpr int NB = D / 16, KS = D / 32, TB = QB / 16;
    constexpr int CB = 2;                       // key / value blocks whose operands are read together
    constexpr int NBUF = 2 * 3 * QB * P * 2 <= 152 * 1024 ? 2 : 1;
    static_assert(TB % 2 == 0, "query slabs are whole MFMA k-steps");
    __shared__ __attribute__((aligned(16))) bf16 sq[NBUF][QB * P];
    __shared__ __attribute__((aligned(16))) bf16 sdh[NBUF][QB * P];    // dnum' hi, or state gradient hi
    __shared__ __attribute__((aligned(16))) bf16 sdl[NBUF][QB * P];    // dnum' lo, or state gradient lo
    __shared__ __attribute__((aligned(16))) double srt[NBUF][QB];      // F_t - m_t of the slab
    __shared__ __attribute__((aligned(16))) float sdd[NBUF][QB];       // dden'_t
    int bh, cb;
    grid_block(in.heads, bh, cb);               // the first key blocks have the most query blocks
    const int tid = threadIdx.x, lane = tid & 63, ln = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int c0 = cb * 64;
    const int s = c0 + 16 * wave + ln;           // this lane's key
    const bool sval = s < S;
    const double Qs = sval ? ws.gk[tokh + s] : 0.0;
    const bf16* dnh_g = reinterpret_cast<const bf16*>(ws.dnum);
    const bf16* dnl_g = dnh_g + (size_t)in.heads * S * dv;

    // two-level form: query blocks of this superchunk only, the later ones through the
    // gradient of the state at the end of this superchunk, weighted by omega_s
    const int sg = c0 / in.LS;
    const int r_hi = min(S, (sg + 1) * in.LS);
    const bf16* Nhi = ss.dC;
    const bf16* Nlo = ss.dC;
    int nsl = 0;
    float omega = 0.0f;
    if (sg < in.G - 1) {
        Nhi = ss.dC + state_off(bh, sg, in.G, dv, dqk);
        Nlo = Nhi + (size_t)dv * dqk;
        nsl = (dv + QB - 1) / QB;
        const int ep = (sg + 1) * in.LS - 1;
        if (sval) omega = exp_arg(ws.F[tokh + ep] - Qs - ws.m[tokh + ep]);
    }
    const int np = nsl + (r_hi - c0 + QB - 1) / QB;

    const DmaOffs<QB, D> ofq(dqk, wave, lane), ofn(dv, wave, lane);
    const unsigned aq = lds_addr(sq), ah = lds_addr(sdh), al = lds_addr(sdl), art = lds_addr(srt), add = lds_addr(sdd);
    constexpr unsigned TILE_B = QB * P * 2;
    auto issue = [&](int p) __attribute__((always_inline)) {
        if (p >= np) return;
        const int b = NBUF == 2 ? (p & 1) : 0;
        if (p < nsl) {
            dma_tile<QB, D>(ah + TILE_B * b, Nhi + (size_t)QB * p * dqk, dv - QB * p, dqk, ofq, wave);
            dma_tile<QB, D>(al + TILE_B * b, Nlo + (size_t)QB * p * dqk, dv - QB * p, dqk, ofq, wave);
        } else {
            const int r0 = c0 + QB * (p - nsl);
            dma_tile<QB, D>(aq + TILE_B * b, in.q + (tokh + r0) * dqk, S - r0, dqk, ofq, wave);
            dma_tile<QB, D>(ah + TILE_B * b, dnh_g + (tokh + r0) * dv, S - r0, dv, ofn, wave);
            dma_tile<QB, D>(al + TILE_B * b, dnl_g + (tokh + r0) * dv, S - r0, dv, ofn, wave);
            const unsigned nq = (unsigned)min(QB, S - r0);
            if (wave == 1) dma_span(art + 8u * QB * b, ws.rt + tokh + r0, 8u * nq, QB / 2, lane);
            if (wave == 2) dma_span(add + 4u * QB * b, ws.dden + tokh + r0, 4u * nq, QB / 4, lane);
        }
    };
    // at item p: wait for its loads and pass a barrier (after which item p - 1, the
    // other set's user, is done everywhere), then issue item p + 1 into that set; with
    // one set, the next item is issued only after this one's products
    auto begin = [&](int p) __attribute__((always_inline)) {
        if constexpr (NBUF == 2) {
            wait_vm<0>();
            __syncthreads();
            issue(p + 1);
        } else {
            if (p > 0) {
                __syncthreads();
                issue(p);
            }
            wait_vm<0>();
            __syncthreads();
        }
    };
    issue(0);

    // k_s and v_s as B operands (k-slot 8g + j <-> dimension 32 kk + 8g + j): held in
    // registers across all query blocks up to width 384; at 512 they do not fit and
    // are re-read (from cache) at every k-step
    constexpr bool KV_REG = D <= 384;
    auto kop = [&](int kk) { return ld8(in.k + (tokh + s) * dqk + 32 * kk + 8 * g, sval && 32 * kk + 8 * g < dqk); };
    auto vop = [&](int kk) { return ld8(in.v + (tokh + s) * dv + 32 * kk + 8 * g, sval && 32 * kk + 8 * g < dv); };
    bf16x8 kb[KV_REG ? KS : 1], vb[KV_REG ? KS : 1];
    if constexpr (KV_REG) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            kb[kk] = kop(kk);
            vb[kk] = vop(kk);
        }
    }
    f32x4 dka[NB], dva[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) dka[b] = dva[b] = f32x4{0, 0, 0, 0};

    // QB-row slices of dC~ (hi, lo):
    //   dv^T[n][s] += dC~[n][j] k_s[j]   (direct reads of the slice's rows n)
    //   dk^T[j][s] += dC~^T[j][n] v_s[n] (transposing reads, n within the slice)
    static_for<D / QB>([&](auto slc) __attribute__((always_inline)) {
        constexpr int sl = decltype(slc)::value;
        if (sl >= nsl) return;
        begin(sl);
        const bf16* th = sdh[NBUF == 2 ? (sl & 1) : 0];
        const bf16* tl_ = sdl[NBUF == 2 ? (sl & 1) : 0];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 kbk = KV_REG ? kb[KV_REG ? kk : 0] : kop(kk);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int off = (16 * tb + ln) * P + 32 * kk + 8 * g;
                dva[TB * sl + tb] = mfma(*reinterpret_cast<const bf16x8*>(th + off), kbk, dva[TB * sl + tb]);
                dva[TB * sl + tb] = mfma(*reinterpret_cast<const bf16x8*>(tl_ + off), kbk, dva[TB * sl + tb]);
            }
        }
#pragma unroll
        for (int kq = 0; kq < QB / 32; ++kq) {
            const int kk = QB / 32 * sl + kq;
            const bf16x8 vbk = KV_REG ? vb[KV_REG ? kk : 0] : vop(kk);
#pragma unroll
            for (int b0 = 0; b0 < NB; b0 += CB) {
                bf16x8 ah[CB], al[CB];
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int off = (32 * kq + 8 * g + (ln >> 2)) * P + 16 * (b0 + j) + 4 * (ln & 3);
                    ah[j] = cat(lds_read_tr(th + off), lds_read_tr(th + off + 4 * P));
                    al[j] = cat(lds_read_tr(tl_ + off), lds_read_tr(tl_ + off + 4 * P));
                }
#pragma unroll
                for (int j = 0; j < CB; ++j) dka[b0 + j] = mfma(ah[j], vbk, dka[b0 + j]);
#pragma unroll
                for (int j = 0; j < CB; ++j) dka[b0 + j] = mfma(al[j], vbk, dka[b0 + j]);
            }
        }
    });
    if (nsl > 0) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            dka[b] *= omega;
            dva[b] *= omega;
        }
    }

    for (int p = nsl; p < np; ++p) {
        const int r0 = c0 + QB * (p - nsl);
        begin(p);
        const int b = NBUF == 2 ? (p & 1) : 0;
        const bf16* tq = sq[b];
        const bf16* th = sdh[b];
        const bf16* tl_ = sdl[b];
        const double* rt = srt[b];
        const float* ddp = sdd[b];
        // S[t][s] and dA[t][s] - dden'_t for the TB query blocks
        f32x4 sc[TB], da[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) sc[tb] = da[tb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            const bf16x8 kbk = KV_REG ? kb[KV_REG ? kk : 0] : kop(kk);
            const bf16x8 vbk = KV_REG ? vb[KV_REG ? kk : 0] : vop(kk);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int off = (16 * tb + ln) * P + 32 * kk + 8 * g;
                sc[tb] = mfma(*reinterpret_cast<const bf16x8*>(tq + off), kbk, sc[tb]);
                da[tb] = mfma(*reinterpret_cast<const bf16x8*>(th + off), vbk, da[tb]);
                da[tb] = mfma(*reinterpret_cast<const bf16x8*>(tl_ + off), vbk, da[tb]);
            }
        }
        // P = S (.) D', G = (dA + dden') (.) D', as hi/lo B operands over query slots
        bf16x8 ph[TB / 2], pl[TB / 2], gh[TB / 2], gl[TB / 2];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = 16 * tb + 4 * g + i;
                const float d = (sval && s <= r0 + tl && r0 + tl < S) ? exp_arg(rt[tl] - Qs) : 0.0f;
                bf16 hi, lo;
                hilo(sc[tb][i] * d, hi, lo);
                ph[tb >> 1][4 * (tb & 1) + i] = hi;
                pl[tb >> 1][4 * (tb & 1) + i] = lo;
                hilo((da[tb][i] + ddp[tl]) * d, hi, lo);
                gh[tb >> 1][4 * (tb & 1) + i] = hi;
                gl[tb >> 1][4 * (tb & 1) + i] = lo;
            }
        // dk^T[j][s] += Q^T G ;  dv^T[n][s] += dnum'^T P.  The operands of CB blocks are
        // read together, then their MFMAs run on independent accumulators.
#pragma unroll
        for (int b0 = 0; b0 < NB; b0 += CB)
#pragma unroll
            for (int pr = 0; pr < TB / 2; ++pr) {
                bf16x8 aq[CB], ah[CB], al[CB];
#pragma unroll
                for (int j = 0; j < CB; ++j) {
                    const int off = (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (b0 + j) + 4 * (ln & 3);
                    aq[j] = cat(lds_read_tr(tq + off), lds_read_tr(tq + off + 16 * P));
                    ah[j] = cat(lds_read_tr(th + off), lds_read_tr(th + off + 16 * P));
                    al[j] = cat(lds_read_tr(tl_ + off), lds_read_tr(tl_ + off + 16 * P));
                }
#pragma unroll
                for (int j = 0; j < CB; ++j) dka[b0 + j] = mfma(aq[j], gh[pr], dka[b0 + j]);
#pragma unroll
                for (int j = 0; j < CB; ++j) dva[b0 + j] = mfma(ah[j], ph[pr], dva[b0 + j]);
#pragma unroll
                for (int j = 0; j < CB; ++j) dka[b0 + j] = mfma(aq[j], gl[pr], dka[b0 + j]);
#pragma unroll
                for (int j = 0; j < CB; ++j) dva[b0 + j] = mfma(ah[j], pl[pr], dva[b0 + j]);
#pragma unroll
                for (int j = 0; j < CB; ++j) dva[b0 + j] = mfma(al[j], ph[pr], dva[b0 + j]);
            }
    }
    // the state gradient's share omega_s dn~, loaded now that no tile loads are in flight
    const float* dnt = ss.dn + ((size_t)bh * (in.G - 1) + (nsl > 0 ? sg : 0)) * dqk;
    float kdk = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int j0 = 16 * b + 4 * g;
        if (sval && j0 < dqk) {
            if (nsl > 0) dka[b] += omega * load4(dnt + j0);
            *reinterpret_cast<f32x4*>(dk + (tokh + s) * dqk + j0) = dka[b];
            const f32x4 k4 = load4(in.k + (tokh + s) * dqk + j0);
#pragma unroll
            for (int i = 0; i < 4; ++i) kdk += k4[i] * dka[b][i];
        }
        if (sval && j0 < dv) *reinterpret_cast<f32x4*>(dvv + (tokh + s) * dv + j0) = dva[b];
    }
    kdk += __shfl_xor(kdk, 16, 64);
    kdk += __shfl_xor(kdk, 32, 64);
    if (sval && g == 0) di[tokh + s] = kdk;
}

// q_t . dq_t (into ws.qdq) and k_t . dk_t (into di) for the paths that do not form
// them in their own passes: one wave per token, 16-byte loads along the feature
// axis, fp64 partial sums
template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_dots_kernel(BwdIn<T> in, BwdWs ws, const float* __restrict__ dq,
                                                              const float* __restrict__ dk, float* __restrict__ di,
                                                              long long tokens)
{
    const int lane = threadIdx.x & 63, dqk = in.dqk;
    for (long long tok = (long long)blockIdx.x * (BW_THREADS / 64) + (threadIdx.x >> 6); tok < tokens;
         tok += (long long)gridDim.x * (BW_THREADS / 64)) {
        double a = 0.0, b = 0.0;
        for (int j = 4 * lane; j < dqk; j += 256) {
            const f32x4 q4 = load4(in.q + tok * dqk + j), g4 = load4(dq + tok * dqk + j);
            const f32x4 k4 = load4(in.k + tok * dqk + j), h4 = load4(dk + tok * dqk + j);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a += (double)q4[i] * g4[i];
                b += (double)k4[i] * h4[i];
            }
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            a += __shfl_xor(a, off, 64);
            b += __shfl_xor(b, off, 64);
        }
        if (lane == 0) {
            ws.qdq[tok] = (float)a;
            di[tok] = (float)b;
        }
    }
}

template <typename T, bool DOTS>
hipError_t launch_gates(const BwdArgs& a, const BwdIn<T>& in, const BwdWs& w) {
    const dim3 sgrid((unsigned)((size_t)a.B * a.NH * ((a.S + GSEG - 1) / GSEG)));
    hipError_t e;
    if constexpr (!DOTS) {
        const long long tokens = (long long)a.B * a.NH * a.S;
        const long long blocks = (tokens + BW_THREADS / 64 - 1) / (BW_THREADS / 64);
        hipLaunchKernelGGL((bwd_dots_kernel<T>), dim3((unsigned)(blocks < (1LL << 20) ? blocks : (1LL << 20))), dim3(BW_THREADS), 0,
                           a.stream, in, w, a.dq, a.dk, a.di, tokens);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_gates_kernel<T>), sgrid, dim3(BW_THREADS), 0, a.stream, in, w, a.di);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gates_fix<T>), sgrid, dim3(BW_THREADS), 0, a.stream, in, w, a.df);
    return hipGetLastError();
}

// smallest tile width covering both dimensions (0 = not on the MFMA path)
int mfma_bwd_width(const BwdArgs& a) {
    if (a.dtype != MLSTM_BF16) return 0;
    const int d = a.dqk > a.dv ? a.dqk : a.dv;
    const int widths[5] = {64, 128, 256, 384, 512};
    for (int i = 0; i < 5; ++i)
        if (d <= widths[i]) return widths[i];
    return 0;
}

template <int D, int QB>
hipError_t launch_bwd_mfma(const BwdArgs& a, const BwdIn<bf16>& in, const BwdWs& w, const SuperStates& ss) {
    const int heads = a.B * a.NH, nb = (a.S + 63) / 64;
    const long long tiles = (long long)((a.dv + LT - 1) / LT) * ((a.dqk + LT - 1) / LT);
    const dim3 lgrid((unsigned)(tiles * heads * (ss.G - 1)));
    const long long quads = (long long)heads * (((long long)a.dv * a.dqk + a.dqk) / 4);
    const dim3 sgrid((unsigned)((quads + WK_THREADS - 1) / WK_THREADS));
    hipError_t e;
    if (ss.G > 1) {
        hipLaunchKernelGGL((bwd_state_local<false>), lgrid, dim3(64 * LW), 0, a.stream, in, w, ss, ss.part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_state_scan<false>), sgrid, dim3(WK_THREADS), 0, a.stream, in, w, ss, ss.part, quads);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_rows_mfma<D>), dim3(heads * nb), dim3(MB_THREADS), 0, a.stream, in, w, ss, a.dq, a.dout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (ss.G > 1) {
        hipLaunchKernelGGL((bwd_state_local<true>), lgrid, dim3(64 * LW), 0, a.stream, in, w, ss, ss.part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_state_scan<true>), sgrid, dim3(WK_THREADS), 0, a.stream, in, w, ss, ss.part, quads);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_cols_mfma<D, QB>), dim3(heads * nb), dim3(MB_THREADS), 0, a.stream, in, w, ss, a.dk,
                       a.dvv, a.di);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_gates<bf16, true>(a, in, w);
}

// ===========================================================================
// GEMM form (bf16, max(d_qk, d_v) > 384): the score-shaped matrices materialized
// ===========================================================================
// Feature widths above 512 do not fit the per-query register tiles of the MFMA
// form above, and at 512 they spill.  For widths above 384 the same quantities (readings of the header) are formed as
// six causal GEMMs over [S_p x S_p] score-shaped matrices held in the workspace
// (S_p = S rounded up to 128; zero above the diagonal and beyond S), each a tiled
// bf16 MFMA product with fp32 accumulation and a fused epilogue:
//   P   = (Q K^T) (.) D'                    (+ row sums = den')       tiles t >= s
//   num'= P V                                                          s < tile end
//   per query: u, do~, dnum', dden'        (bwd_gemm_query)
//   G   = (dnum' V^T + dden') (.) D'                                   tiles t >= s
//   dq  = G K,   dk = G^T Q,   dv = P^T dnum'
// P, G and dnum' are computed values and enter their products as bf16 hi + lo.
constexpr int GT = 128;                  // output tile, rows and columns
constexpr int GK = 32;                   // k per step (one MFMA depth)
constexpr int GTHREADS = 256;            // 2 x 2 waves, 64 x 64 each
constexpr int GPR = GK + 8;              // LDS pitch of [row][k] tiles (bf16)
constexpr int GPT = GT + 16;             // LDS pitch of [k][row] tiles: 8 banks mod 64 between rows, so the
                                         // transposing reads (4 rows x 4 8-byte chunks per 16 lanes) never collide

enum GLayout { ROWK = 0, KROW = 1 };     // stored [row][k] (k contiguous) or [k][row]
enum GEpi { EPI_F32 = 0, EPI_P = 1, EPI_G = 2 };
enum GKRange { K_FULL = 0, K_UPTO = 1, K_FROM = 2 };   // k in [0,K), [0, tile end), [tile start, K)

struct GOp {
    const bf16* hi;
    const bf16* lo;          // null for an exact operand
    long long ld, hs;        // row stride and head stride, elements
    int rows;                // valid rows (m or n); a multiple of 8 for KROW
    int kv;                  // valid k; a multiple of 8 for ROWK
};

struct GEpiArgs {
    float* out; long long ldo, hso; int Mv, Nv;       // EPI_F32
    bf16* mat;                                         // EPI_P / EPI_G: P or G (hi; lo at + heads Sp^2)
    float* rowpart;                                    // EPI_P
    int S, Sp, heads;
};

template <int L>
struct GTileSize { static constexpr int N = L == ROWK ? GT * GPR : GK * GPT; };

// this thread's two 16-byte units of a 128 x 32 operand tile (global -> registers)
template <int L>
__device__ __forceinline__ void g_load(bf16x8 (&r)[2], const bf16* base, const GOp& op, int r0, int k0, int tid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = tid + GTHREADS * u;
        if constexpr (L == ROWK) {
            const int row = id >> 2, k8 = 8 * (id & 3);
            r[u] = ld8(base + (long long)(r0 + row) * op.ld + k0 + k8, r0 + row < op.rows && k0 + k8 < op.kv);
        } else {
            const int kr = id >> 4, c8 = 8 * (id & 15);
            r[u] = ld8(base + (long long)(k0 + kr) * op.ld + r0 + c8, k0 + kr < op.kv && r0 + c8 < op.rows);
        }
    }
}
template <int L>
__device__ __forceinline__ void g_store(const bf16x8 (&r)[2], bf16* tile, int tid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int id = tid + GTHREADS * u;
        if constexpr (L == ROWK) *reinterpret_cast<bf16x8*>(tile + (id >> 2) * GPR + 8 * (id & 3)) = r[u];
        else *reinterpret_cast<bf16x8*>(tile + (id >> 4) * GPT + 8 * (id & 15)) = r[u];
    }
}
// MFMA operand (16 rows w0 + 16 b .. + 15, k-slots 8g .. 8g + 7 of the step)
template <int L>
__device__ __forceinline__ bf16x8 g_operand(const bf16* tile, int w0, int b, int ln, int g) {
    if constexpr (L == ROWK) {
        return *reinterpret_cast<const bf16x8*>(tile + (w0 + 16 * b + ln) * GPR + 8 * g);
    } else {
        const bf16* p = tile + (8 * g + (ln >> 2)) * GPT + w0 + 16 * b + 4 * (ln & 3);
        return cat(lds_read_tr(p), lds_read_tr(p + 4 * GPT));
    }
}

template <int LA, int LB, bool ALO, bool BLO>
struct alignas(16) GemmSmem {
    bf16 a[2][ALO ? 2 : 1][GTileSize<LA>::N];
    bf16 b[2][BLO ? 2 : 1][GTileSize<LB>::N];
};

// One workgroup per (output tile, head).  TRI: only tiles with tn <= tm (the
// causal lower triangle), enumerated in a 1-D grid; otherwise tiles in rows of
// Nt, ordered so the ones with most k steps start first.
template <int LA, int LB, bool ALO, bool BLO, int EPI, int KR, bool TRI>
__global__ __launch_bounds__(GTHREADS) void bwd_gemm(GOp A, GOp B, int M, int N, int K, GEpiArgs ep, BwdWs ws,
                                                     BwdIn<bf16> in)
{
    __shared__ GemmSmem<LA, LB, ALO, BLO> sm;
    // Workgroups are dealt to the 8 XCDs round robin; renumber them so each XCD
    // takes a contiguous run of the (head, tile) order, whose neighbouring tiles
    // share operand rows in that XCD's L2.
    const unsigned total = gridDim.x * gridDim.y;
    unsigned lin = blockIdx.x + blockIdx.y * gridDim.x;
    if (total % 8 == 0) lin = (lin % 8) * (total / 8) + lin / 8;
    const int bh = (int)(lin / gridDim.x), bid = (int)(lin % gridDim.x);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;
    const int Mt = (M + GT - 1) / GT, Nt = (N + GT - 1) / GT;
    int tm, tn;
    if constexpr (TRI) {
        const int idx = bid;
        tm = (int)((sqrtf(8.0f * idx + 1.0f) - 1.0f) * 0.5f);
        while ((long long)tm * (tm + 1) / 2 > idx) --tm;
        while ((long long)(tm + 1) * (tm + 2) / 2 <= idx) ++tm;
        tn = idx - tm * (tm + 1) / 2;
    } else {
        const int row = bid / Nt;
        tn = bid % Nt;
        tm = KR == K_UPTO ? Mt - 1 - row : row;        // most k steps first
    }
    const int m0 = GT * tm, n0 = GT * tn;
    const int wm = 64 * (wave >> 1), wn = 64 * (wave & 1);
    const int k_begin = KR == K_FROM ? m0 : 0;
    const int k_end = KR == K_UPTO ? min(K, m0 + GT) : K;
    const bf16* ah = A.hi + (long long)bh * A.hs;
    const bf16* al = ALO ? A.lo + (long long)bh * A.hs : nullptr;
    const bf16* bhp = B.hi + (long long)bh * B.hs;
    const bf16* blp = BLO ? B.lo + (long long)bh * B.hs : nullptr;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

    bf16x8 rah[2], ral[2], rbh[2], rbl[2];
    auto load = [&](int k0) {
        g_load<LA>(rah, ah, A, m0, k0, tid);
        if constexpr (ALO) g_load<LA>(ral, al, A, m0, k0, tid);
        g_load<LB>(rbh, bhp, B, n0, k0, tid);
        if constexpr (BLO) g_load<LB>(rbl, blp, B, n0, k0, tid);
    };
    auto store = [&](int buf) {
        g_store<LA>(rah, sm.a[buf][0], tid);
        if constexpr (ALO) g_store<LA>(ral, sm.a[buf][1], tid);
        g_store<LB>(rbh, sm.b[buf][0], tid);
        if constexpr (BLO) g_store<LB>(rbl, sm.b[buf][1], tid);
    };
    if (k_begin < k_end) {
        load(k_begin);
        store(0);
        __syncthreads();
    }
    for (int k0 = k_begin; k0 < k_end; k0 += GK) {
        const int cur = ((k0 - k_begin) / GK) & 1;
        const bool more = k0 + GK < k_end;
        if (more) load(k0 + GK);                       // in flight during the products
        bf16x8 bo[4], bol[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bo[j] = g_operand<LB>(sm.b[cur][0], wn, j, ln, g);
            if constexpr (BLO) bol[j] = g_operand<LB>(sm.b[cur][1], wn, j, ln, g);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 ao = g_operand<LA>(sm.a[cur][0], wm, i, ln, g);
            bf16x8 aol;
            if constexpr (ALO) aol = g_operand<LA>(sm.a[cur][1], wm, i, ln, g);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc[i][j] = mfma(ao, bo[j], acc[i][j]);
                if constexpr (ALO) acc[i][j] = mfma(aol, bo[j], acc[i][j]);
                if constexpr (BLO) acc[i][j] = mfma(ao, bol[j], acc[i][j]);
            }
        }
        if (more) store(cur ^ 1);                      // the other buffer, free since the last barrier
        __syncthreads();
    }

    // epilogue: lane holds rows m0 + wm + 16 i + 4 g + e, column n0 + wn + 16 j + ln
    const long long hsq = (long long)ep.Sp * ep.Sp;
    if constexpr (EPI == EPI_F32) {
        float* o = ep.out + (long long)bh * ep.hso;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = m0 + wm + 16 * i + 4 * g + e;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn + 16 * j + ln;
                    if (m < ep.Mv && n < ep.Nv) o[(long long)m * ep.ldo + n] = acc[i][j][e];
                }
            }
    } else {
        // P = S (.) D' or G = (dA + dden'_t) (.) D', with D'_ts = exp(F_t - m_t - (F_s - i~_s))
        // for s <= t < S and 0 elsewhere (also beyond S, so the products can read whole tiles)
        const size_t tokh = (size_t)bh * ep.S;
        bf16* mh = ep.mat + (long long)bh * hsq;
        bf16* ml = mh + (long long)ep.heads * hsq;
        double qs[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = n0 + wn + 16 * j + ln;
            qs[j] = s < ep.S ? ws.F[tokh + s] - (double)in.i_pre[tokh + s] : 0.0;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = m0 + wm + 16 * i + 4 * g + e;
                const bool tv = t < ep.S;
                const double rt = tv ? ws.F[tokh + t] - ws.m[tokh + t] : 0.0;
                const float add = (EPI == EPI_G && tv) ? ws.dden[tokh + t] : 0.0f;
                float rsum = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s = n0 + wn + 16 * j + ln;
                    const float d = (tv && s <= t) ? exp_arg(rt - qs[j]) : 0.0f;
                    const float v = (acc[i][j][e] + add) * d;
                    rsum += v;
                    bf16 hi, lo;
                    hilo(v, hi, lo);
                    mh[(long long)t * ep.Sp + s] = hi;
                    ml[(long long)t * ep.Sp + s] = lo;
                }
                if constexpr (EPI == EPI_P) {
                    // sum over the 16 lanes of the row, then one partial per (row, wave column)
#pragma unroll
                    for (int off = 8; off > 0; off >>= 1) rsum += __shfl_xor(rsum, off, 64);
                    if (ln == 0 && tv)
                        ep.rowpart[(tokh + t) * (2 * ep.Sp / GT) + 2 * tn + (wave & 1)] = rsum;
                }
            }
    }
}

// Per query t: den' from the row partials, then u, do~, dnum' (bf16 hi, lo) and dden',
// with the arithmetic of the MFMA form's per-query phase.
__global__ __launch_bounds__(BW_THREADS) void bwd_gemm_query(BwdIn<bf16> in, BwdWs ws, GemmWs gw,
                                                            float* __restrict__ dout)
{
    __shared__ float red[BW_THREADS / 64];
    __shared__ float bc;
    const int t = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = in.S, dv = in.dv;
    const size_t tok = (size_t)bh * S + t;
    const int np = 2 * (t / GT + 1);                   // row partials of the tiles at or left of t's
    if (wave == 0) {
        float x = 0.0f;
        for (int i = lane; i < np; i += 64) x += gw.rowpart[tok * (2 * gw.Sp / GT) + i];
        x = wave_sum(x);
        if (lane == 0) bc = x;
    }
    __syncthreads();
    const float den = bc;
    const float fl = exp_arg(-ws.m[tok]);
    const float rN = 1.0f / fmaxf(fabsf(den), fl);
    const float* nump = gw.num + tok * dv;
    const float* op = in.o_pre + tok * dv;
    const bf16* dhp = in.dh + tok * dv;
    bf16* dnh = reinterpret_cast<bf16*>(ws.dnum) + tok * dv;
    bf16* dnl = dnh + (size_t)in.heads * S * dv;
    float duu = 0.0f;
    for (int n = 4 * tid; n < dv; n += 4 * BW_THREADS) {
        const f32x4 nm = load4(nump + n), o4 = load4(op + n), dh4 = load4(dhp + n);
        f32x4 do4;
        bf16x4 h4, l4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float u = nm[i] * rN;
            const float gg = sigmoid(o4[i]);
            do4[i] = dh4[i] * u * gg * (1.0f - gg);
            const float du = dh4[i] * gg;
            duu += du * u;
            bf16 hi, lo;
            hilo(du * rN, hi, lo);
            h4[i] = hi;
            l4[i] = lo;
        }
        *reinterpret_cast<f32x4*>(dout + tok * dv + n) = do4;
        *reinterpret_cast<bf16x4*>(dnh + n) = h4;
        *reinterpret_cast<bf16x4*>(dnl + n) = l4;
    }
    duu = wave_sum(duu);
    if (lane == 0) red[wave] = duu;
    __syncthreads();
    if (tid == 0) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < BW_THREADS / 64; ++w) s += red[w];
        ws.dden[tok] = fabsf(den) > fl ? -(den > 0.0f ? 1.0f : -1.0f) * s * rN : 0.0f;
    }
}

template <int LA, int LB, bool ALO, bool BLO, int EPI, int KR, bool TRI>
hipError_t launch_gemm(const BwdArgs& a, const GOp& A, const GOp& B, int M, int N, int K, const GEpiArgs& ep,
                       const BwdWs& w, const BwdIn<bf16>& in) {
    const int Mt = (M + GT - 1) / GT, Nt = (N + GT - 1) / GT;
    const unsigned tiles = TRI ? (unsigned)(Mt * (Mt + 1) / 2) : (unsigned)(Mt * Nt);
    hipLaunchKernelGGL((bwd_gemm<LA, LB, ALO, BLO, EPI, KR, TRI>), dim3(tiles, a.B * a.NH), dim3(GTHREADS), 0,
                       a.stream, A, B, M, N, K, ep, w, in);
    return hipGetLastError();
}

hipError_t launch_bwd_gemm(const BwdArgs& a, const BwdIn<bf16>& in, const BwdWs& w, const GemmWs& gw) {
    const int heads = a.B * a.NH, S = a.S, Sp = gw.Sp, dqk = a.dqk, dv = a.dv;
    const long long hsq = (long long)Sp * Sp;
    const bf16* q = in.q; const bf16* k = in.k; const bf16* v = in.v;
    const bf16* dnh = reinterpret_cast<const bf16*>(w.dnum);
    const bf16* dnl = dnh + (size_t)heads * S * dv;
    GEpiArgs ep = {};
    ep.S = S; ep.Sp = Sp; ep.heads = heads;
    hipError_t e;
    // P = (Q K^T) (.) D' and its row sums
    {
        GOp A = {q, nullptr, dqk, (long long)S * dqk, S, dqk};
        GOp B = {k, nullptr, dqk, (long long)S * dqk, S, dqk};
        GEpiArgs p = ep; p.mat = gw.P; p.rowpart = gw.rowpart;
        if ((e = launch_gemm<ROWK, ROWK, false, false, EPI_P, K_FULL, true>(a, A, B, Sp, Sp, dqk, p, w, in)) != hipSuccess) return e;
    }
    // num' = P V
    {
        GOp A = {gw.P, gw.P + heads * hsq, Sp, hsq, Sp, Sp};
        GOp B = {v, nullptr, dv, (long long)S * dv, dv, S};
        GEpiArgs o = ep; o.out = gw.num; o.ldo = dv; o.hso = (long long)S * dv; o.Mv = S; o.Nv = dv;
        if ((e = launch_gemm<ROWK, KROW, true, false, EPI_F32, K_UPTO, false>(a, A, B, S, dv, Sp, o, w, in)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(bwd_gemm_query, dim3(S, heads), dim3(BW_THREADS), 0, a.stream, in, w, gw, a.dout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // G = (dnum' V^T + dden') (.) D'
    {
        GOp A = {dnh, dnl, dv, (long long)S * dv, S, dv};
        GOp B = {v, nullptr, dv, (long long)S * dv, S, dv};
        GEpiArgs p = ep; p.mat = gw.G;
        if ((e = launch_gemm<ROWK, ROWK, true, false, EPI_G, K_FULL, true>(a, A, B, Sp, Sp, dv, p, w, in)) != hipSuccess) return e;
    }
    // dq = G K
    {
        GOp A = {gw.G, gw.G + heads * hsq, Sp, hsq, Sp, Sp};
        GOp B = {k, nullptr, dqk, (long long)S * dqk, dqk, S};
        GEpiArgs o = ep; o.out = a.dq; o.ldo = dqk; o.hso = (long long)S * dqk; o.Mv = S; o.Nv = dqk;
        if ((e = launch_gemm<ROWK, KROW, true, false, EPI_F32, K_UPTO, false>(a, A, B, S, dqk, Sp, o, w, in)) != hipSuccess) return e;
    }
    // dk = G^T Q
    {
        GOp A = {gw.G, gw.G + heads * hsq, Sp, hsq, Sp, Sp};
        GOp B = {q, nullptr, dqk, (long long)S * dqk, dqk, S};
        GEpiArgs o = ep; o.out = a.dk; o.ldo = dqk; o.hso = (long long)S * dqk; o.Mv = S; o.Nv = dqk;
        if ((e = launch_gemm<KROW, KROW, true, false, EPI_F32, K_FROM, false>(a, A, B, S, dqk, Sp, o, w, in)) != hipSuccess) return e;
    }
    // dv = P^T dnum'
    {
        GOp A = {gw.P, gw.P + heads * hsq, Sp, hsq, Sp, Sp};
        GOp B = {dnh, dnl, dv, (long long)S * dv, dv, S};
        GEpiArgs o = ep; o.out = a.dvv; o.ldo = dv; o.hso = (long long)S * dv; o.Mv = S; o.Nv = dv;
        if ((e = launch_gemm<KROW, KROW, true, true, EPI_F32, K_FROM, false>(a, A, B, S, dv, Sp, o, w, in)) != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a) {
    const int heads = a.B * a.NH;
    BwdWs w;
    SuperStates ss;
    GemmWs gw;
    bwd_ws_walk((char*)a.ws, a, &w, &ss, &gw);
    BwdIn<T> in;
    in.q = (const T*)a.q; in.k = (const T*)a.k; in.v = (const T*)a.v; in.dh = (const T*)a.dh;
    in.i_pre = a.i_pre; in.f_pre = a.f_pre; in.o_pre = a.o_pre;
    in.S = a.S; in.dqk = a.dqk; in.dv = a.dv;
    const int nb = (a.S + BT - 1) / BT;
    in.heads = heads;
    in.nb = nb;
    in.LS = ss.LS;
    in.G = ss.G;
    const dim3 sgrid((unsigned)((size_t)heads * ((a.S + GSEG - 1) / GSEG)));
    hipLaunchKernelGGL(bwd_gate_local, sgrid, dim3(BW_THREADS), 0, a.stream, a.i_pre, a.f_pre, a.S, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_gate_fix, sgrid, dim3(BW_THREADS), 0, a.stream, a.i_pre, a.S, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (sizeof(T) == 2) {
        if (bwd_gemm_path(a)) {
            if ((e = launch_bwd_gemm(a, in, w, gw)) != hipSuccess) return e;
            return launch_gates<bf16, false>(a, in, w);
        }
        switch (mfma_bwd_width(a)) {
            case 64: return launch_bwd_mfma<64, 64>(a, in, w, ss);
            case 128: return launch_bwd_mfma<128, 64>(a, in, w, ss);
            case 256: return launch_bwd_mfma<256, 32>(a, in, w, ss);
            case 384: return launch_bwd_mfma<384, 32>(a, in, w, ss);
            case 512: return launch_bwd_mfma<512, 32>(a, in, w, ss);
            default: break;
        }
    }
    hipLaunchKernelGGL((bwd_rows_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dq, a.dout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_cols_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dk, a.dvv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_gates<T, false>(a, in, w);
}

}  // namespace

size_t bwd_workspace_bytes(const BwdArgs& a) {
    return bwd_ws_walk(nullptr, a, nullptr, nullptr, nullptr);
}

hipError_t launch_bwd(const BwdArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_bwd_t<bf16>(a);
    return launch_bwd_t<float>(a);
}

}  // namespace mlstm
