// C ABI of libmlstm: argument validation and kernel dispatch.
// The operations are defined in include/mlstm.h ("xLSTM: Extended Long
// Short-Term Memory", sections 2.2 and 2.3).  Nothing here computes: every
// step of the cell runs in the HIP kernels this file launches.
#include <stdarg.h>
#include <stdio.h>

#include "mlstm_internal.h"

namespace {

thread_local char g_detail[512] = "";

mlstm_status fail(mlstm_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return s;
}

mlstm_status ok() {
    g_detail[0] = '\0';
    return MLSTM_OK;
}

constexpr int MAX_DIM = 4096;

bool aligned(const void* p, unsigned a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool aligned16(const void* p) { return aligned(p, 16); }

mlstm_status check_dims(int dqk, int dv) {
    if (dqk < 16 || dqk > MAX_DIM || dqk % 16 != 0)
        return fail(MLSTM_ERR_INVALID_ARG, "d_qk=%d must be a multiple of 16 in [16, %d]", dqk, MAX_DIM);
    if (dv < 16 || dv > MAX_DIM || dv % 16 != 0)
        return fail(MLSTM_ERR_INVALID_ARG, "d_v=%d must be a multiple of 16 in [16, %d]", dv, MAX_DIM);
    return MLSTM_OK;
}

mlstm_status check_dtype(mlstm_dtype dt) {
    if (dt != MLSTM_F32 && dt != MLSTM_BF16)
        return fail(MLSTM_ERR_INVALID_ARG, "dtype=%d is neither MLSTM_F32 nor MLSTM_BF16", (int)dt);
    return MLSTM_OK;
}

// validates everything except pointers and workspace; fills a (sizes only)
mlstm_status check_fwd_sizes(int B, int NH, int S, int dqk, int dv, int chunk, mlstm_dtype dt) {
    if (B < 1 || NH < 1 || S < 1)
        return fail(MLSTM_ERR_INVALID_ARG, "B=%d, NH=%d, S=%d must all be >= 1", B, NH, S);
    mlstm_status s = check_dims(dqk, dv);
    if (s != MLSTM_OK) return s;
    if ((s = check_dtype(dt)) != MLSTM_OK) return s;
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return fail(MLSTM_ERR_INVALID_ARG, "chunk=%d must be 16, 32, 64 or 128", chunk);
    if (S % chunk != 0)
        return fail(MLSTM_ERR_INVALID_ARG, "S=%d is not a multiple of chunk=%d", S, chunk);
    const long long heads = (long long)B * NH;
    if (heads > 65535LL * 64)
        return fail(MLSTM_ERR_UNSUPPORTED, "B*NH=%lld exceeds the supported number of heads", heads);
    const long long elems = heads * S * (long long)(dqk > dv ? dqk : dv);
    if (elems > (1LL << 40))
        return fail(MLSTM_ERR_UNSUPPORTED, "tensor of %lld elements is too large", elems);
    return MLSTM_OK;
}

mlstm::FwdArgs make_fwd_args(int B, int NH, int S, int dqk, int dv, int chunk, mlstm_dtype dt) {
    mlstm::FwdArgs a = {};
    a.B = B; a.NH = NH; a.S = S; a.dqk = dqk; a.dv = dv; a.chunk = chunk; a.dtype = dt;
    return a;
}

size_t fwd_ws_bytes(const mlstm::FwdArgs& a) {
    if (a.dtype == MLSTM_BF16 && mlstm::mfma_fwd_supported(a)) return mlstm::mfma_fwd_workspace_bytes(a);
    return mlstm::valu_fwd_workspace_bytes(a);
}

}  // namespace

extern "C" {

size_t mlstm_fwd_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype) {
    if (check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype) != MLSTM_OK) return 0;
    return fwd_ws_bytes(make_fwd_args(B, NH, S, d_qk, d_v, chunk, dtype));
}

// Validates the forward's arguments and fills a; stage bits: 1 = prepare, 2 = scan.
static mlstm_status fwd_common(const void* q, const void* k, const void* v,
                               const float* i_pre, const float* f_pre, const float* o_pre,
                               int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                               void* h_out, float* C_final, float* n_final, float* m_final,
                               void* workspace, size_t workspace_bytes, void* stream, int stages) {
    mlstm_status s = check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype);
    if (s != MLSTM_OK) return s;
    // tensors read or written with vector accesses need 16-byte alignment, the others their element size
    const void* ptrs[] = {q, k, v, i_pre, f_pre, o_pre, h_out, C_final, n_final, m_final};
    const char* names[] = {"q", "k", "v", "i_pre", "f_pre", "o_pre", "h_out", "C_final", "n_final", "m_final"};
    const unsigned align[] = {16, 16, 16, 4, 4, 16, 16, 16, 16, 4};
    for (int p = 0; p < 10; ++p) {
        // prepare alone reads only q, k and the two scalar gates
        const bool needed = (stages & 2) || p == 0 || p == 1 || p == 3 || p == 4;
        if (!needed) continue;
        if (!ptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", names[p]);
        if (!aligned(ptrs[p], align[p]))
            return fail(MLSTM_ERR_INVALID_ARG, "%s is not %u-byte aligned", names[p], align[p]);
    }
    mlstm::FwdArgs a = make_fwd_args(B, NH, S, d_qk, d_v, chunk, dtype);
    a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
    a.h = h_out; a.C = C_final; a.n = n_final; a.m = m_final;
    a.C0 = nullptr; a.n0 = nullptr; a.m0 = nullptr;
    const size_t need = fwd_ws_bytes(a);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(MLSTM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
        if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    a.ws = workspace; a.ws_bytes = workspace_bytes;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    const bool two_stage = dtype == MLSTM_BF16 && mlstm::mfma_fwd_supported(a);
    hipError_t e = hipSuccess;
    if (two_stage) {
        if (stages & 1) e = mlstm::launch_fwd_mfma_prepare(a);
        if (e == hipSuccess && (stages & 2)) e = mlstm::launch_fwd_mfma_scan(a);
    } else if (stages & 2) {
        e = mlstm::launch_fwd_valu(a);
    }
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mlstm_status mlstm_fwd_parallel(const void* q, const void* k, const void* v,
                                const float* i_pre, const float* f_pre, const float* o_pre,
                                int B, int NH, int S, int d_qk, int d_v, int chunk,
                                mlstm_dtype dtype,
                                void* h_out, float* C_final, float* n_final, float* m_final,
                                void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype,
                      h_out, C_final, n_final, m_final, workspace, workspace_bytes, stream, 3);
}

mlstm_status mlstm_fwd_prepare(const void* q, const void* k, const float* i_pre, const float* f_pre,
                               int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, nullptr, i_pre, f_pre, nullptr, B, NH, S, d_qk, d_v, chunk, dtype,
                      nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, 1);
}

mlstm_status mlstm_fwd_scan(const void* q, const void* k, const void* v,
                            const float* i_pre, const float* f_pre, const float* o_pre,
                            int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                            void* h_out, float* C_final, float* n_final, float* m_final,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype,
                      h_out, C_final, n_final, m_final, workspace, workspace_bytes, stream, 2);
}

mlstm_status mlstm_step(const void* q, const void* k, const void* v,
                        const float* i_pre, const float* f_pre, const float* o_pre,
                        int B, int NH, int d_qk, int d_v, mlstm_dtype dtype,
                        float* C, float* n, float* m, void* h_out, void* stream) {
    if (B < 1 || NH < 1) return fail(MLSTM_ERR_INVALID_ARG, "B=%d, NH=%d must be >= 1", B, NH);
    mlstm_status s = check_dims(d_qk, d_v);
    if (s != MLSTM_OK) return s;
    if ((s = check_dtype(dtype)) != MLSTM_OK) return s;
    if ((long long)B * NH > 0x7fffffffLL) return fail(MLSTM_ERR_UNSUPPORTED, "B*NH too large");
    // q, k, C and n are read with vector accesses; the rest element by element
    const unsigned el = dtype == MLSTM_BF16 ? 2u : 4u;
    const void* ptrs[] = {q, k, v, i_pre, f_pre, o_pre, C, n, m, h_out};
    const char* names[] = {"q", "k", "v", "i_pre", "f_pre", "o_pre", "C", "n", "m", "h_out"};
    const unsigned align[] = {16, 16, el, 4, 4, 4, 16, 16, 4, el};
    for (int p = 0; p < 10; ++p) {
        if (!ptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", names[p]);
        if (!aligned(ptrs[p], align[p]))
            return fail(MLSTM_ERR_INVALID_ARG, "%s is not %u-byte aligned", names[p], align[p]);
    }
    mlstm::StepArgs a = {};
    a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
    a.B = B; a.NH = NH; a.dqk = d_qk; a.dv = d_v; a.dtype = dtype;
    a.C = C; a.n = n; a.m = m; a.h = h_out;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = mlstm::launch_step(a);
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char* mlstm_status_string(mlstm_status status) {
    switch (status) {
        case MLSTM_OK: return "ok";
        case MLSTM_ERR_INVALID_ARG: return "invalid argument";
        case MLSTM_ERR_UNSUPPORTED: return "unsupported configuration";
        case MLSTM_ERR_WORKSPACE: return "workspace missing or too small";
        case MLSTM_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* mlstm_error_detail(void) { return g_detail; }

}  // extern "C"
