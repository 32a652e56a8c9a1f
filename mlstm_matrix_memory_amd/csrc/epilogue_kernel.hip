// mLSTM block epilogue: per-head GroupNorm of the cell output, learnable skip,
// external output gate ("xLSTM: Extended Long Short-Term Memory", Figure 10 and
// its caption, the mLSTM block).
//
// For every (batch, head, token) row of d_v channels:
//   mu = mean(h),  var = mean((h - mu)^2)
//   y  = (gn_w (.) (h - mu) / sqrt(var + eps) + gn_b + skip_w (.) x) (.) act(z)
// with per-channel parameters of the head and act = sigmoid or swish.
//
// One wave per row.  The row is read once into registers (4 channels per lane per
// 16-channel group of the wave's 64-lane sweep), mean and variance are two
// register passes with wave reductions (no second read of h), then x, z and the
// parameters are read and y written with the same vector accesses.  The kernel
// is bound by HBM: per row it reads h, x, z and writes y once.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

constexpr int EP_THREADS = 256;     // 4 rows per workgroup

__device__ __forceinline__ void store4(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// CPL: 4-channel chunks per lane (d_v <= 256 * CPL)
template <typename T, int CPL>
__global__ __launch_bounds__(EP_THREADS) void epilogue_kernel(
    const T* __restrict__ h, const T* __restrict__ x, const T* __restrict__ z,
    const float* __restrict__ gn_w, const float* __restrict__ gn_b, const float* __restrict__ skip_w,
    long long rows, int NH, int S, int dv, float eps, int act, T* __restrict__ y)
{
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * (EP_THREADS / 64) + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int head = (int)((row / S) % NH);
    const size_t base = (size_t)row * dv;
    const int nch = dv / 4;
    f32x4 hv[CPL];
    float sum = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        hv[c] = ch < nch ? load4(h + base + 4 * ch) : f32x4{0, 0, 0, 0};
        sum += (hv[c][0] + hv[c][1]) + (hv[c][2] + hv[c][3]);
    }
    const float mu = wave_sum(sum) / dv;
    float sq = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = hv[c][i] - mu;
                sq += e * e;
            }
        }
    }
    const float rstd = 1.0f / sqrtf(wave_sum(sq) / dv + eps);
    const float* pw = gn_w + (size_t)head * dv;
    const float* pb = gn_b + (size_t)head * dv;
    const float* ps = skip_w + (size_t)head * dv;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
            const f32x4 xv = load4(x + base + 4 * ch), zv = load4(z + base + 4 * ch);
            const f32x4 w4 = load4(pw + 4 * ch), b4 = load4(pb + 4 * ch), s4 = load4(ps + 4 * ch);
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = sigmoid(zv[i]);
                const float g = act == 0 ? sg : zv[i] * sg;
                o[i] = (w4[i] * (hv[c][i] - mu) * rstd + b4[i] + s4[i] * xv[i]) * g;
            }
            store4(y + base + 4 * ch, o);
        }
    }
}

template <typename T>
hipError_t launch_epilogue_t(const EpilogueArgs& a) {
    const long long rows = (long long)a.B * a.NH * a.S;
    const int cpl = (a.dv / 4 + 63) / 64;
    const dim3 grid((unsigned)((rows + EP_THREADS / 64 - 1) / (EP_THREADS / 64)));
    const T* h = (const T*)a.h; const T* x = (const T*)a.x; const T* z = (const T*)a.z;
    T* y = (T*)a.y;
#define EP_CASE(N)                                                                                          \
    if (cpl <= N) {                                                                                         \
        hipLaunchKernelGGL((epilogue_kernel<T, N>), grid, dim3(EP_THREADS), 0, a.stream, h, x, z, a.gn_w, \
                           a.gn_b, a.skip_w, rows, a.NH, a.S, a.dv, a.eps, a.act, y);                      \
        return hipGetLastError();                                                                           \
    }
    EP_CASE(1)
    EP_CASE(2)
    EP_CASE(4)
    EP_CASE(8)
    EP_CASE(16)
#undef EP_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_epilogue(const EpilogueArgs& a) {
    if (a.dtype == MLSTM_BF16) return launch_epilogue_t<bf16>(a);
    return launch_epilogue_t<float>(a);
}

}  // namespace mlstm
