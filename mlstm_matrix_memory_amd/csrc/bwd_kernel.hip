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
    float* dnum;    // [heads][S][dv] num' while it accumulates, then dnum' (vector-ALU path);
                    // the MFMA path keeps dnum' there as bf16 hi [heads][S][dv], then lo
    float* dden;    // [heads][S] dden'
    float* qdq;     // [heads][S] q_t . dq_t (MFMA path)
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
    w.qdq = (float*)take(heads * S * sizeof(float));
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
    int heads, nb;          // heads and 64-token blocks per head
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
// di~_j = k_j . dk_j ;  dF_j = q_j . dq_j - k_j . dk_j ;  df~_j = sigmoid(-f~_j) sum_{t>=j} dF_t
// DOTS: q . dq comes from the workspace and k . dk is already in di (MFMA path)
template <typename T, bool DOTS>
__global__ __launch_bounds__(BW_THREADS) void bwd_gates_kernel(BwdIn<T> in, const float* __restrict__ dq,
                                                               const float* __restrict__ dk,
                                                               const float* __restrict__ qdq_in,
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
            if (DOTS) {
                dF = (double)qdq_in[tokh + t] - (double)di[tokh + t];
            } else {
                double qdq = 0.0, kdk = 0.0;
                for (int j = 0; j < dqk; ++j) {
                    qdq += (double)to_f32(in.q[(tokh + t) * dqk + j]) * dq[(tokh + t) * dqk + j];
                    kdk += (double)to_f32(in.k[(tokh + t) * dqk + j]) * dk[(tokh + t) * dqk + j];
                }
                di[tokh + t] = (float)kdk;
                dF = qdq - kdk;
            }
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

// K and V rows [row0, row0 + 64) into LDS (pitch P) with every load of both tiles
// issued before the first store: one memory round trip per stage instead of one per
// batch.  (Used up to width 384, where the 2 * D / 32 registers per thread fit beside
// the live state; wider tiles go through stage_rows in batches.)
template <int D, int P>
__device__ __forceinline__ void stage_kv(bf16* dk_, bf16* dv_, const bf16* ks, const bf16* vs, size_t tok0,
                                         int row0, int S, int dqk, int dv, int tid) {
    constexpr int UPT = 64 * D / 8 / MB_THREADS;
    bf16x8 rk[UPT], rv[UPT];
#pragma unroll
    for (int b = 0; b < UPT; ++b) {
        const int u = tid + b * MB_THREADS;
        const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
        rk[b] = ld8(ks + (tok0 + row0 + r) * dqk + c8, row0 + r < S && c8 < dqk);
        rv[b] = ld8(vs + (tok0 + row0 + r) * dv + c8, row0 + r < S && c8 < dv);
    }
#pragma unroll
    for (int b = 0; b < UPT; ++b) {
        const int u = tid + b * MB_THREADS;
        const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
        *reinterpret_cast<bf16x8*>(dk_ + r * P + c8) = rk[b];
        *reinterpret_cast<bf16x8*>(dv_ + r * P + c8) = rv[b];
    }
}

// Q, dnum' hi and dnum' lo rows [row0, row0 + R) into LDS with every load issued
// before the first store (one memory round trip per stage)
template <int R, int D, int P>
__device__ __forceinline__ void stage_qd(bf16* dq_, bf16* dh_, bf16* dl_, const bf16* qs, const bf16* hs,
                                         const bf16* ls, size_t tok0, int row0, int S, int dqk, int dv, int tid) {
    constexpr int UPT = R * D / 8 / MB_THREADS;
    bf16x8 rq[UPT], rh[UPT], rl[UPT];
#pragma unroll
    for (int b = 0; b < UPT; ++b) {
        const int u = tid + b * MB_THREADS;
        const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
        rq[b] = ld8(qs + (tok0 + row0 + r) * dqk + c8, row0 + r < S && c8 < dqk);
        rh[b] = ld8(hs + (tok0 + row0 + r) * dv + c8, row0 + r < S && c8 < dv);
        rl[b] = ld8(ls + (tok0 + row0 + r) * dv + c8, row0 + r < S && c8 < dv);
    }
#pragma unroll
    for (int b = 0; b < UPT; ++b) {
        const int u = tid + b * MB_THREADS;
        const int r = u / (D / 8), c8 = 8 * (u % (D / 8));
        *reinterpret_cast<bf16x8*>(dq_ + r * P + c8) = rq[b];
        *reinterpret_cast<bf16x8*>(dh_ + r * P + c8) = rh[b];
        *reinterpret_cast<bf16x8*>(dl_ + r * P + c8) = rl[b];
    }
}

template <int D>
struct alignas(16) RowsSmem {
    bf16 k[64 * (D + 8)];
    bf16 v[64 * (D + 8)];
    double gs[64];       // F_s - i~_s of the key block
};

// per (head, query block of 64): num', den' over key blocks <= it, then dnum', dden',
// do~ (wave-local), then dq over the same key blocks, and q_t . dq_t
template <int D>
__global__ __launch_bounds__(MB_THREADS) void bwd_rows_mfma(BwdIn<bf16> in, BwdWs ws, float* __restrict__ dq,
                                                          float* __restrict__ dout)
{
    constexpr int P = D + 8;
    constexpr int NB = D / 16, KS = D / 32;
    constexpr int GB = 4;                       // value / key blocks whose operands are read together
    static_assert(NB % GB == 0, "width must be a multiple of 64");
    __shared__ RowsSmem<D> sm;
    int bh, rb;
    grid_block(in.heads, bh, rb);
    rb = in.nb - 1 - rb;                        // the last query blocks have the most key blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int r0 = rb * 64;
    const int t = r0 + 16 * wave + ln;          // this lane's query
    const bool tval = t < S;
    const double Rt = tval ? ws.F[tokh + t] - ws.m[tokh + t] : 0.0;
    const float fl = tval ? exp_arg(-ws.m[tokh + t]) : 1.0f;

    // q_t as B operands: k-slot 8g + j <-> key dimension 32 kk + 8g + j
    bf16x8 qb[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qb[kk] = ld8(in.q + (tokh + t) * dqk + 32 * kk + 8 * g, tval && 32 * kk + 8 * g < dqk);

    auto stage = [&](int c0) {
        __syncthreads();
        if constexpr (D <= 384) {
            stage_kv<D, P>(sm.k, sm.v, in.k, in.v, tokh, c0, S, dqk, dv, tid);
        } else {
            stage_rows<64, D, P, 8>(sm.k, in.k, tokh, c0, S, dqk, tid);
            stage_rows<64, D, P, 8>(sm.v, in.v, tokh, c0, S, dv, tid);
        }
        if (tid < 64) {
            const int s = min(c0 + tid, S - 1);
            sm.gs[tid] = ws.F[tokh + s] - (double)in.i_pre[tokh + s];
        }
        __syncthreads();
    };
    // D'[s][t] for this lane's 16 entries of a tile pair (s = 16 sb + 4g + i)
    auto decay4 = [&](float (&d)[4][4], int c0) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 16 * sb + 4 * g + i;
                d[sb][i] = (tval && c0 + sl <= t) ? exp_arg(Rt - sm.gs[sl]) : 0.0f;
            }
    };

    // ---- pass 1: num'^T[n][t] and den_t -------------------------------------
    f32x4 num[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) num[nb] = f32x4{0, 0, 0, 0};
    float den = 0.0f;
    for (int cb = 0; cb <= rb; ++cb) {
        const int c0 = 64 * cb;
        stage(c0);
        f32x4 st[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) st[sb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int k0 = 0; k0 < KS; k0 += 2) {
            bf16x8 a[2][4];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    a[j][sb] = k0 + j < KS ? *reinterpret_cast<const bf16x8*>(sm.k + (16 * sb + ln) * P + 32 * (k0 + j) + 8 * g)
                                           : bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    if (k0 + j < KS) st[sb] = mfma(a[j][sb], qb[k0 + j < KS ? k0 + j : 0], st[sb]);
        }
        float d[4][4];
        decay4(d, c0);
        bf16x8 ph[2], pl[2];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = st[sb][i] * d[sb][i];
                den += p;
                bf16 hi, lo;
                hilo(p, hi, lo);
                ph[sb >> 1][4 * (sb & 1) + i] = hi;
                pl[sb >> 1][4 * (sb & 1) + i] = lo;
            }
        // operands of GB value blocks read together, then their products with
        // consecutive MFMAs on independent accumulators (LDS latency overlaps)
#pragma unroll
        for (int nb0 = 0; nb0 < NB; nb0 += GB) {
            bf16x8 a[GB][2];
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const bf16* vp = sm.v + (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (nb0 + j) + 4 * (ln & 3);
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
    for (int cb = 0; cb <= rb; ++cb) {
        const int c0 = 64 * cb;
        stage(c0);
        f32x4 da[4];
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) da[sb] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int pr = 0; pr < NB / 2; ++pr) {
            bf16x8 a[4];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const bf16* vp = sm.v + (16 * sb + ln) * P + 32 * pr + 4 * g;
                a[sb] = cat(*reinterpret_cast<const bf16x4*>(vp), *reinterpret_cast<const bf16x4*>(vp + 16));
            }
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) da[sb] = mfma(a[sb], dnh[pr], da[sb]);
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) da[sb] = mfma(a[sb], dnl[pr], da[sb]);
        }
        float d[4][4];
        decay4(d, c0);
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
#pragma unroll
        for (int jb0 = 0; jb0 < NB; jb0 += GB) {
            bf16x8 a[GB][2];
#pragma unroll
            for (int j = 0; j < GB; ++j)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const bf16* kp = sm.k + (32 * pr + 4 * g + (ln >> 2)) * P + 16 * (jb0 + j) + 4 * (ln & 3);
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
    float qdq = 0.0f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
        const int j0 = 16 * jb + 4 * g;
        if (tval && j0 < dqk) {
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

template <int D, int QB>
struct alignas(16) ColsSmem {
    bf16 q[QB * (D + 8)];
    bf16 dh[QB * (D + 8)];      // dnum' hi
    bf16 dl[QB * (D + 8)];      // dnum' lo
    double rt[QB];              // F_t - m_t of the query block
    float dd[QB];               // dden'_t
};

// per (head, key block of 64): dk, dv over query blocks >= it (QB queries at a
// time), and k_s . dk_s (= di~_s)
template <int D, int QB>
__global__ __launch_bounds__(MB_THREADS) void bwd_cols_mfma(BwdIn<bf16> in, BwdWs ws, float* __restrict__ dk,
                                                          float* __restrict__ dvv, float* __restrict__ di)
{
    constexpr int P = D + 8;
    constexpr int NB = D / 16, KS = D / 32, TB = QB / 16;
    constexpr int CB = 2;                       // key / value blocks whose operands are read together
    __shared__ ColsSmem<D, QB> sm;
    int bh, cb;
    grid_block(in.heads, bh, cb);               // the first key blocks have the most query blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, ln = lane & 15, g = lane >> 4;
    const int S = in.S, dqk = in.dqk, dv = in.dv;
    const size_t tokh = (size_t)bh * S;
    const int c0 = cb * 64;
    const int s = c0 + 16 * wave + ln;           // this lane's key
    const bool sval = s < S;
    const double Qs = sval ? ws.F[tokh + s] - (double)in.i_pre[tokh + s] : 0.0;
    const bf16* dnh_g = reinterpret_cast<const bf16*>(ws.dnum);
    const bf16* dnl_g = dnh_g + (size_t)in.heads * S * dv;

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

    for (int r0 = c0; r0 < S; r0 += QB) {
        __syncthreads();
        if constexpr (QB * D <= 32 * 384) {
            stage_qd<QB, D, P>(sm.q, sm.dh, sm.dl, in.q, dnh_g, dnl_g, tokh, r0, S, dqk, dv, tid);
        } else {
            stage_rows<QB, D, P, 4>(sm.q, in.q, tokh, r0, S, dqk, tid);
            stage_rows<QB, D, P, 4>(sm.dh, dnh_g, tokh, r0, S, dv, tid);
            stage_rows<QB, D, P, 4>(sm.dl, dnl_g, tokh, r0, S, dv, tid);
        }
        if (tid < QB) {
            const int tt = min(r0 + tid, S - 1);
            sm.rt[tid] = ws.F[tokh + tt] - ws.m[tokh + tt];
            sm.dd[tid] = r0 + tid < S ? ws.dden[tokh + tt] : 0.0f;
        }
        __syncthreads();
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
                sc[tb] = mfma(*reinterpret_cast<const bf16x8*>(sm.q + off), kbk, sc[tb]);
                da[tb] = mfma(*reinterpret_cast<const bf16x8*>(sm.dh + off), vbk, da[tb]);
                da[tb] = mfma(*reinterpret_cast<const bf16x8*>(sm.dl + off), vbk, da[tb]);
            }
        }
        // P = S (.) D', G = (dA + dden') (.) D', as hi/lo B operands over query slots
        bf16x8 ph[TB / 2], pl[TB / 2], gh[TB / 2], gl[TB / 2];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tl = 16 * tb + 4 * g + i;
                const float d = (sval && s <= r0 + tl && r0 + tl < S) ? exp_arg(sm.rt[tl] - Qs) : 0.0f;
                bf16 hi, lo;
                hilo(sc[tb][i] * d, hi, lo);
                ph[tb >> 1][4 * (tb & 1) + i] = hi;
                pl[tb >> 1][4 * (tb & 1) + i] = lo;
                hilo((da[tb][i] + sm.dd[tl]) * d, hi, lo);
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
                    aq[j] = cat(lds_read_tr(sm.q + off), lds_read_tr(sm.q + off + 16 * P));
                    ah[j] = cat(lds_read_tr(sm.dh + off), lds_read_tr(sm.dh + off + 16 * P));
                    al[j] = cat(lds_read_tr(sm.dl + off), lds_read_tr(sm.dl + off + 16 * P));
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
    float kdk = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const int j0 = 16 * b + 4 * g;
        if (sval && j0 < dqk) {
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
hipError_t launch_bwd_mfma(const BwdArgs& a, const BwdIn<bf16>& in, const BwdWs& w) {
    const int heads = a.B * a.NH, nb = (a.S + 63) / 64;
    hipLaunchKernelGGL((bwd_rows_mfma<D>), dim3(heads * nb), dim3(MB_THREADS), 0, a.stream, in, w, a.dq, a.dout);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_cols_mfma<D, QB>), dim3(heads * nb), dim3(MB_THREADS), 0, a.stream, in, w, a.dk, a.dvv,
                       a.di);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gates_kernel<bf16, true>), dim3(heads), dim3(BW_THREADS), 0, a.stream, in, a.dq, a.dk,
                       w.qdq, a.di, a.df);
    return hipGetLastError();
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
    in.heads = heads;
    in.nb = nb;
    hipLaunchKernelGGL(bwd_gate_kernel, dim3(heads), dim3(BW_THREADS), 0, a.stream, a.i_pre, a.f_pre, a.S, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (sizeof(T) == 2) {
        switch (mfma_bwd_width(a)) {
            case 64: return launch_bwd_mfma<64, 64>(a, in, w);
            case 128: return launch_bwd_mfma<128, 64>(a, in, w);
            case 256: return launch_bwd_mfma<256, 64>(a, in, w);
            case 384: return launch_bwd_mfma<384, 32>(a, in, w);
            case 512: return launch_bwd_mfma<512, 32>(a, in, w);
            default: break;
        }
    }
    hipLaunchKernelGGL((bwd_rows_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dq, a.dout);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_cols_kernel<T>), dim3(heads, nb), dim3(BW_THREADS), 0, a.stream, in, w, a.dk, a.dvv);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_gates_kernel<T, false>), dim3(heads), dim3(BW_THREADS), 0, a.stream, in, a.dq, a.dk,
                       nullptr, a.di, a.df);
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
