// Column padding for the matrix-core forward.
//
// "xLSTM: Extended Long Short-Term Memory", section 2.3, eq. (18) and the
// normalizer after it: q and k enter the cell only through contractions over the
// key dimension (the scores q.k, the state update v k^T and its normalizer n,
// and the retrievals C q and n.q).  A key column that is zero in both q and k
// therefore adds exact zeros to every one of them, and the state columns it
// would own stay zero.  The matrix-core forward has tilings for key widths that
// are multiples of 64; a bf16 forward of another width up to 1024 runs on copies
// of q and k (and of a given initial C' and n') widened with zero columns, and
// the final C' and n' are narrowed back.  This file only moves bytes.
#include "mlstm_internal.h"

namespace mlstm {
namespace {

struct alignas(16) Unit16 {
    unsigned w[4];
};

// dst[r][u] = src[r][u] for u < src_units, zero for src_units <= u < dst_units
// (padding), or dst[r][u] = src[r][u] for u < dst_units <= src_units (narrowing).
// Each thread moves UPT units spaced one grid apart, all loads issued before the
// stores, so that several loads are in flight per thread; I is the index type
// (32-bit whenever the unit count fits).
constexpr int UPT = 4;

template <class U, class I>
__global__ __launch_bounds__(256) void copy_cols_kernel(const U* __restrict__ src, U* __restrict__ dst, I n,
                                                        int src_units, int dst_units) {
    const I stride = (I)gridDim.x * blockDim.x;
    for (I base = (I)blockIdx.x * blockDim.x + threadIdx.x; base < n; base += stride * UPT) {
        U val[UPT];
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const I i = base + (I)j * stride;
            val[j] = U{};
            if (i < n) {
                const I r = i / (I)dst_units;
                const int u = (int)(i - r * (I)dst_units);
                if (u < src_units) val[j] = src[r * (I)src_units + u];
            }
        }
#pragma unroll
        for (int j = 0; j < UPT; ++j) {
            const I i = base + (I)j * stride;
            if (i < n) dst[i] = val[j];
        }
    }
}

template <class U>
hipError_t launch_copy(const void* src, void* dst, size_t rows, size_t src_row_bytes, size_t dst_row_bytes,
                       hipStream_t stream) {
    const int su = (int)(src_row_bytes / sizeof(U)), du = (int)(dst_row_bytes / sizeof(U));
    const size_t n = rows * (size_t)du;
    if (n == 0) return hipSuccess;
    const size_t want = (n + 256 * UPT - 1) / (256 * UPT);
    const unsigned blocks = (unsigned)(want < 16384 ? want : 16384);
    // 32-bit indices when every index fits: the source's as well (larger when
    // narrowing), and the loop's, which runs up to a grid stride past the end
    const size_t src_n = rows * (size_t)su;
    if ((n > src_n ? n : src_n) + (size_t)blocks * 256 * UPT < ((size_t)1 << 32))
        hipLaunchKernelGGL((copy_cols_kernel<U, unsigned>), dim3(blocks), dim3(256), 0, stream, (const U*)src,
                           (U*)dst, (unsigned)n, su, du);
    else
        hipLaunchKernelGGL((copy_cols_kernel<U, size_t>), dim3(blocks), dim3(256), 0, stream, (const U*)src,
                           (U*)dst, n, su, du);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_cols(const void* src, void* dst, size_t rows, size_t src_row_bytes, size_t dst_row_bytes,
                            hipStream_t stream) {
    const bool wide = (src_row_bytes % 16 == 0) && (dst_row_bytes % 16 == 0) &&
                      ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) == 0;
    if (wide) return launch_copy<Unit16>(src, dst, rows, src_row_bytes, dst_row_bytes, stream);
    if (src_row_bytes % 4 != 0 || dst_row_bytes % 4 != 0 ||
        ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 3) != 0)
        return hipErrorInvalidValue;
    return launch_copy<unsigned>(src, dst, rows, src_row_bytes, dst_row_bytes, stream);
}

}  // namespace mlstm
