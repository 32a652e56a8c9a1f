// mLSTM block epilogue: per-head GroupNorm of the cell output, learnable skip,
// external output gate ("xLSTM: Extended Long Short-Term Memory", Figure 10 and
// its caption, the mLSTM block).
//
// For every (batch, head, token) row of d_v channels:
//   mu = mean(h),  var = mean((h - mu)^2)
//   y  = (gn_w (.) (h - mu) / sqrt(var + eps) + gn_b + skip_w (.) x) (.) act(z)
// with per-channel parameters of the head and act = sigmoid or swish.
//
// One row per group of 16, 32 or 64 lanes (by d_v).  The row is read once into
// registers in 8-channel chunks, mean and variance are two register passes with
// reductions over the group (no second read of h), then x, z and the parameters
// are read and y written with the same 16-byte accesses.  The kernel is bound by
// HBM: per row it reads h, x, z and writes y once.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int EP_THREADS = 256;

typedef __attribute__((ext_vector_type(8))) float f32x8;

__device__ __forceinline__ f32x8 load8(const float* p) {
    const f32x4 a = load4(p), b = load4(p + 4);
    return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 load8(const bf16* p) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
    f32x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (float)v[e];
    return r;
}
__device__ __forceinline__ void store8(float* p, f32x8 v) {
    *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8(bf16* p, f32x8 v) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (bf16)v[e];
    *reinterpret_cast<bf16x8*>(p) = r;
}

// sum over the G lanes of a row group (G = 16, 32 or 64 consecutive lanes)
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// One row per group of G lanes (64 / G rows per wave); CPL 8-channel chunks per lane
// (d_v <= 8 * G * CPL), read and written with 16-byte (bf16) or 32-byte (fp32) accesses.
template <typename T, int G, int CPL>
__global__ __launch_bounds__(EP_THREADS) void epilogue_kernel(
    const T* __restrict__ h, const T* __restrict__ x, const T* __restrict__ z,
    const float* __restrict__ gn_w, const float* __restrict__ gn_b, const float* __restrict__ skip_w,
    long long rows, int NH, int S, int dv, float eps, int act, T* __restrict__ y)
{
    const int gl = threadIdx.x % G;
    const long long row = (long long)blockIdx.x * (EP_THREADS / G) + threadIdx.x / G;
    const bool live = row < rows;                      // whole groups are live or not
    const int head = live ? (int)((row / S) % NH) : 0;
    const size_t base = live ? (size_t)row * dv : 0;
    const int nch = dv / 8;
    f32x8 hv[CPL];
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = gl + G * c;
        hv[c] = (live && ch < nch) ? load8(h + base + 8 * ch) : f32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += hv[c][e];
    }
    const float mu = group_sum<G>(sum) / dv;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = gl + G * c;
        if (ch < nch) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float d = hv[c][e] - mu;
                sq += d * d;
            }
        }
    }
    const float rstd = 1.0f / sqrtf(group_sum<G>(sq) / dv + eps);
    if (!live) return;
    const float* pw = gn_w + (size_t)head * dv;
    const float* pb = gn_b + (size_t)head * dv;
    const float* ps = skip_w + (size_t)head * dv;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = gl + G * c;
        if (ch < nch) {
            const f32x8 xv = load8(x + base + 8 * ch), zv = load8(z + base + 8 * ch);
            const f32x8 w8 = load8(pw + 8 * ch), b8 = load8(pb + 8 * ch), s8 = load8(ps + 8 * ch);
            f32x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float sg = sigmoid(zv[e]);
                const float gt = act == 0 ? sg : zv[e] * sg;
                o[e] = (w8[e] * (hv[c][e] - mu) * rstd + b8[e] + s8[e] * xv[e]) * gt;
            }
            store8(y + base + 8 * ch, o);
        }
    }
}

template <typename T>
hipError_t launch_epilogue_t(const EpilogueArgs& a) {
    const long long rows = (long long)a.B * a.NH * a.S;
    const int nch = a.dv / 8;
    const T* h = (const T*)a.h; const T* x = (const T*)a.x; const T* z = (const T*)a.z;
    T* y = (T*)a.y;
#define EP_CASE(G, N)                                                                                          \
    if (nch <= (G) * (N)) {                                                                                    \
        const dim3 grid((unsigned)((rows + EP_THREADS / (G) - 1) / (EP_THREADS / (G))));                       \
        hipLaunchKernelGGL((epilogue_kernel<T, G, N>), grid, dim3(EP_THREADS), 0, a.stream, h, x, z, a.gn_w,  \
                           a.gn_b, a.skip_w, rows, a.NH, a.S, a.dv, a.eps, a.act, y);                         \
        return hipGetLastError();                                                                              \
    }
    EP_CASE(16, 1)      // d_v <= 128: 16 rows per workgroup
    EP_CASE(16, 2)
    EP_CASE(16, 4)      // d_v <= 512
    EP_CASE(32, 4)      // d_v <= 1024
    EP_CASE(64, 4)
    EP_CASE(64, 8)      // d_v <= 4096
#undef EP_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_epilogue(const EpilogueArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_epilogue_t<bf16>(a);
    return launch_epilogue_t<float>(a);
}

}  // namespace mlstm
