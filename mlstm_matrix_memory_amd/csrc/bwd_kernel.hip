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
// Three tiled passes over 64-token blocks, all VALU with fp32 accumulation and
// fp64 exponent arguments:
//   bwd_gate_kernel   per head: F and m (prefix sum, prefix max), fp64
//   bwd_rows_kernel   per (query block, head): num', den' over key blocks <= it, then
//                     dnum', dden', do~; then dq over the same key blocks
//   bwd_cols_kernel   per (key block, head): dk, dv over query blocks >= it
//   bwd_gates_kernel  per head: di~, df~ (reverse prefix sum)
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int BT = 64;           // tokens per block (rows and columns of a score tile)
constexpr int BK = 32;           // contraction slab
constexpr int BW_THREADS = 256;  // 16 x 16 threads, each a 4 x 4 piece of a 64 x 64 tile

struct BwdWs {
    double* F;      // [heads][S] cumulative log forget gate
    double* m;      // [heads][S] stabilizer
    float* dnum;    // [heads][S][dv] num' while it accumulates, then dnum'
    float* dden;    // [heads][S] dden'
};

inline size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t bwd_ws_walk(char* base, size_t heads, size_t S, int dv, BwdWs* out) {
    size_t off = 0;
    auto take = [&](size_t bytes) { char* p = base + off; off += a256(bytes); return p; };
    BwdWs w;
    w.F = (double*)take(heads * S * sizeof(double));
    w.m = (double*)take(heads * S * sizeof(double));
    w.dnum = (float*)take(heads * S * dv * sizeof(float));
    w.dden = (float*)take(heads * S * sizeof(float));
    if (out) *out = w;
    return off;
}

// ---- kernel 1: F and m per head --------------------------------------------
// m_t = max(log f_t + m_{t-1}, i~_t) from m = 0 unrolls to F_t + max(0, max_{s<=t}(i~_s - F_s)).
__global__ __launch_bounds__(BW_THREADS) void bwd_gate_kernel(const float* __restrict__ i_pre,
                                                              const float* __restrict__ f_pre, int S, BwdWs ws)
{
    __shared__ double part[BW_THREADS / 64];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const size_t base = (size_t)bh * S;
    double carry_sum = 0.0, carry_max = 0.0;     // max(0, ...) folds the zero initial state in
    for (int t0 = 0; t0 < S; t0 += BW_THREADS) {
        const int t = t0 + tid;
        double x = t < S ? log_sigmoid_f64((double)f_pre[base + t]) : 0.0;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) part[wave] = x;
        __syncthreads();
        double pre = carry_sum;
        for (int w2 = 0; w2 < wave; ++w2) pre += part[w2];
        const double F = pre + x;
        double tot = carry_sum;
        for (int w2 = 0; w2 < BW_THREADS / 64; ++w2) tot += part[w2];
        __syncthreads();
        double z = t < S ? (double)i_pre[base + t] - F : -INFINITY;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double y = __shfl_up(z, off, 64);
            if (lane >= off) z = fmax(z, y);
        }
        if (lane == 63) part[wave] = z;
        __syncthreads();
        double pm = carry_max;
        for (int w2 = 0; w2 < wave; ++w2) pm = fmax(pm, part[w2]);
        const double M = fmax(pm, z);
        double tm = carry_max;
        for (int w2 = 0; w2 < BW_THREADS / 64; ++w2) tm = fmax(tm, part[w2]);
        __syncthreads();
        if (t < S) {
            ws.F[base + t] = F;
            ws.m[base + t] = F + M;
        }
        carry_sum = tot;
        carry_max = tm;
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
};

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
// di~_j = k_j . dk_j ;  dF_j = q_j . dq_j - k_j . dk_j ;  df~_j = sigmoid(-f~_j) sum_{t>=j} dF_t
template <typename T>
__global__ __launch_bounds__(BW_THREADS) void bwd_gates_kernel(BwdIn<T> in, const float* __restrict__ dq,
                                                               const float* __restrict__ dk,
                                                               float* __restrict__ di, float* __restrict__ df)
{
    __shared__ double part[BW_THREADS / 64];
    const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int S = in.S, dqk = in.dqk;
    const size_t tokh = (size_t)bh * S;
    double carry = 0.0;
    // walk the sequence from the end; within a tile, thread tid holds token end - tid
    for (int e0 = S - 1; e0 >= 0; e0 -= BW_THREADS) {
        const int t = e0 - tid;
        double dF = 0.0;
        if (t >= 0) {
            double qdq = 0.0, kdk = 0.0;
            for (int j = 0; j < dqk; ++j) {
                qdq += (double)to_f32(in.q[(tokh + t) * dqk + j]) * dq[(tokh + t) * dqk + j];
                kdk += (double)to_f32(in.k[(tokh + t) * dqk + j]) * dk[(tokh + t) * dqk + j];
            }
            di[tokh + t] = (float)kdk;
            dF = qdq - kdk;
        }
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
        if (t >= 0) {
            const double f = (double)in.f_pre[tokh + t];
            df[tokh + t] = (float)((pre + x) / (1.0 + exp(f)));    // sigmoid(-f) = 1 / (1 + e^f)
        }
        carry = tot;
    }
}

template <typename T>
hipError_t launch_bwd_t(const BwdArgs& a) {
    const int heads = a.B * a.NH;
    BwdWs w;
    bwd_ws_walk((char*)a.ws, (size_t)heads, a.S, a.dv, &w);
    BwdIn<T> in;
    in.q = (const T*)a.q; in.k = (const T*)a.k; in.v = (const T*)a.v; in.dh = (const T*)a.dh;
    in.i_pre = a.i_pre; in.f_pre = a.f_pre; in.o_pre = a.o_pre;
    in.S = a.S; in.dqk = a.dqk; in.dv = a.dv;
    const int nb = (a.S + BT - 1) / BT;
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(heads), dim3(BW_THREADS), 0, a.stream, a.i_pre, a.f_pre, a.S, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_rows_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dq, a.dout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_cols_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dk, a.dvv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gates_kernel<T>), dim3(heads), dim3(BW_THREADS), 0, a.stream, in, a.dq, a.dk, a.di, a.df);
    return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(const BwdArgs& a) {
    return bwd_ws_walk(nullptr, (size_t)a.B * a.NH, a.S, a.dv, nullptr);
}

hipError_t launch_bwd(const BwdArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_bwd_t<bf16>(a);
    return launch_bwd_t<float>(a);
}

}  // namespace mlstm
