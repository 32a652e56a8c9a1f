// C ABI of libmlstm: argument validation and kernel dispatch.
// The operations are defined in include/mlstm.h ("xLSTM: Extended Long
// Short-Term Memory", sections 2.2 and 2.3).  Nothing here computes: every
// step of the cell runs in the HIP kernels this file launches.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

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

// validates everything except pointers and workspace
mlstm_status check_fwd_sizes(int B, int NH, int S, int dqk, int dv, int chunk, mlstm_dtype dt, bool ragged_ok) {
    if (B < 1 || NH < 1 || S < 1)
        return fail(MLSTM_ERR_INVALID_ARG, "B=%d, NH=%d, S=%d must all be >= 1", B, NH, S);
    mlstm_status s = check_dims(dqk, dv);
    if (s != MLSTM_OK) return s;
    if ((s = check_dtype(dt)) != MLSTM_OK) return s;
    if (chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128)
        return fail(MLSTM_ERR_INVALID_ARG, "chunk=%d must be 16, 32, 64 or 128", chunk);
    if (!ragged_ok && S % chunk != 0)
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
    a.B = B; a.NH = NH; a.S = S; a.Sx = S; a.t_begin = 0; a.dqk = dqk; a.dv = dv; a.chunk = chunk; a.dtype = dt;
    return a;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// How a forward over S tokens runs: the longest multiple of the chunk the bf16
// MFMA path executes (see mfma_fwd_chunk) on that path when it covers the shape,
// the rest (a ragged tail, or everything on the fp32 path and on shapes the MFMA
// path does not cover) on the VALU kernel.  Between the two, the state passes
// through the workspace.  A bf16 key width below 1024 that is not a multiple of
// 64 runs on the MFMA path at the next multiple of 64, from zero-padded copies of
// q and k (and of a given C'_0 and n'_0) in the workspace; zero key columns add
// nothing to any product of the cell, and the final C' and n' are narrowed back.
constexpr int KEY_PAD = 64;
constexpr int KEY_PAD_MAX = 1024;

struct FwdPlan {
    int S_main;             // tokens on the MFMA path (0 = none)
    bool tail;              // the VALU kernel runs over [S_main, S)
    int dq_run;             // key width the MFMA path runs at (d_qk, or d_qk padded)
    bool pad;               // dq_run > d_qk: the MFMA path runs on padded copies
    size_t main_bytes;      // workspace of the MFMA path
    size_t qk_bytes;        // one padded copy of q or k (whole sequences)
    size_t cpad_bytes;      // one padded C' (initial or final)
    size_t npad_bytes;      // one padded n' (initial or final)
    size_t pad_bytes;       // all padded copies
    size_t mid_bytes;       // state handed from the MFMA path to the tail
    size_t total() const { return align256(main_bytes) + pad_bytes + mid_bytes; }
};

FwdPlan plan_fwd(int B, int NH, int S, int dqk, int dv, int chunk, mlstm_dtype dt) {
    FwdPlan pl = {};
    pl.dq_run = dqk;
    const int dq_run = (dt == MLSTM_BF16 && dqk % KEY_PAD != 0 && dqk < KEY_PAD_MAX)
                           ? (dqk + KEY_PAD - 1) / KEY_PAD * KEY_PAD : dqk;
    const int L = mlstm::mfma_fwd_chunk(make_fwd_args(B, NH, S, dq_run, dv, chunk, dt));
    const int S_main = L > 0 ? S - S % L : 0;
    mlstm::FwdArgs a = make_fwd_args(B, NH, S_main, dq_run, dv, chunk, dt);
    const size_t heads = (size_t)B * NH;
    if (S_main > 0 && dt == MLSTM_BF16 && mlstm::mfma_fwd_supported(a)) {
        pl.S_main = S_main;
        pl.main_bytes = mlstm::mfma_fwd_workspace_bytes(a);
        pl.dq_run = dq_run;
        pl.pad = dq_run != dqk;
    }
    if (pl.pad) {
        pl.qk_bytes = align256(heads * (size_t)S * pl.dq_run * 2);
        pl.cpad_bytes = align256(heads * (size_t)dv * pl.dq_run * 4);
        pl.npad_bytes = align256(heads * (size_t)pl.dq_run * 4);
        pl.pad_bytes = 2 * pl.qk_bytes + 2 * (pl.cpad_bytes + pl.npad_bytes);
    }
    pl.tail = pl.S_main < S;
    if (pl.tail && pl.S_main > 0) {
        pl.mid_bytes = align256(heads * dv * dqk * 4) + align256(heads * dqk * 4) + align256(heads * 4);
    }
    return pl;
}

bool overlaps(const void* p, size_t pb, const void* q, size_t qb) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + qb && b < a + pb;
}

// A buffer of a call: its address, size in bytes and name (null or empty = absent).
struct Buf {
    const void* p;
    size_t bytes;
    const char* name;
};

// Every buffer the call writes (the first n_out of `bufs`) must share no byte with
// any other buffer of the call: the kernels read inputs after writing outputs of
// earlier chunks or rows, so an alias would corrupt results without an error.
mlstm_status check_disjoint(const Buf* bufs, int n, int n_out) {
    for (int o = 0; o < n_out; ++o) {
        if (!bufs[o].p || bufs[o].bytes == 0) continue;
        for (int i = 0; i < n; ++i) {
            if (i == o || !bufs[i].p || bufs[i].bytes == 0) continue;
            if (overlaps(bufs[o].p, bufs[o].bytes, bufs[i].p, bufs[i].bytes))
                return fail(MLSTM_ERR_INVALID_ARG, "%s overlaps %s", bufs[o].name, bufs[i].name);
        }
    }
    return MLSTM_OK;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward (mlstm_fwd_parallel_noalloc)
// ---------------------------------------------------------------------------
// One file-scope device array per GPU, held until the process ends.  In host code
// the name `scratch` is only a stand-in for the symbol: its device address, which
// differs per GPU, is looked up once per device with hipGetSymbolAddress and only
// that address is ever handed to kernels.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)160 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of this GPU's scratch array (the current device), or an error.
mlstm_status scratch_for_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= MAX_DEVICES)
        return fail(MLSTM_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", dev,
                    MAX_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(MLSTM_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MLSTM_OK;
}

}  // namespace

extern "C" {

size_t mlstm_fwd_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype) {
    if (check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype, true) != MLSTM_OK) return 0;
    return plan_fwd(B, NH, S, d_qk, d_v, chunk, dtype).total();
}

// The block epilogue's inputs when the scan applies it itself (h_out then receives y).
struct EpiIn {
    const void* x; const void* z;
    const float* gw; const float* gb; const float* sw;
    float eps; int act;
};

// Validates the forward's arguments and launches it; stage bits: 1 = prepare, 2 = scan
// (the staged entry points require S to be a multiple of chunk and the zero initial state).
static mlstm_status fwd_common(const void* q, const void* k, const void* v,
                               const float* i_pre, const float* f_pre, const float* o_pre,
                               int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                               const float* C_init, const float* n_init, const float* m_init,
                               void* h_out, float* C_final, float* n_final, float* m_final,
                               void* workspace, size_t workspace_bytes, void* stream, int stages,
                               bool ragged_ok, const EpiIn* ep = nullptr) {
    mlstm_status s = check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype, ragged_ok);
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
    const size_t heads = (size_t)B * NH;
    const int given = (C_init != nullptr) + (n_init != nullptr) + (m_init != nullptr);
    if (given != 0 && given != 3)
        return fail(MLSTM_ERR_INVALID_ARG, "C_init, n_init and m_init must be given together (or all NULL)");
    if (given == 3) {
        if (!aligned16(C_init)) return fail(MLSTM_ERR_INVALID_ARG, "C_init is not 16-byte aligned");
        if (!aligned(n_init, 4) || !aligned(m_init, 4))
            return fail(MLSTM_ERR_INVALID_ARG, "n_init / m_init are not 4-byte aligned");
        const void* in[] = {C_init, n_init, m_init};
        const size_t inb[] = {heads * d_v * d_qk * 4, heads * d_qk * 4, heads * 4};
        const void* out[] = {C_final, n_final, m_final};
        for (int i = 0; i < 3; ++i)
            for (int o = 0; o < 3; ++o)
                if (overlaps(in[i], inb[i], out[o], inb[o]))
                    return fail(MLSTM_ERR_INVALID_ARG, "the initial state overlaps the final state");
    }
    const FwdPlan pl = plan_fwd(B, NH, S, d_qk, d_v, chunk, dtype);
    const size_t need = pl.total();
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(MLSTM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
        if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    {
        // outputs first: the workspace, h and the final state are written
        const size_t el = dtype == MLSTM_BF16 ? 2 : 4;
        const size_t tok = heads * (size_t)S;
        const bool scan = (stages & 2) != 0;
        const Buf bufs[] = {
            {need > 0 ? workspace : nullptr, need, "workspace"},
            {scan ? h_out : nullptr, tok * d_v * el, "h_out"},
            {scan ? C_final : nullptr, heads * d_v * d_qk * 4, "C_final"},
            {scan ? n_final : nullptr, heads * d_qk * 4, "n_final"},
            {scan ? m_final : nullptr, heads * 4, "m_final"},
            {q, tok * d_qk * el, "q"}, {k, tok * d_qk * el, "k"},
            {scan ? v : nullptr, tok * d_v * el, "v"},
            {i_pre, tok * 4, "i_pre"}, {f_pre, tok * 4, "f_pre"},
            {scan ? o_pre : nullptr, tok * d_v * 4, "o_pre"},
            {C_init, heads * d_v * d_qk * 4, "C_init"}, {n_init, heads * d_qk * 4, "n_init"},
            {m_init, heads * 4, "m_init"},
        };
        if ((s = check_disjoint(bufs, (int)(sizeof(bufs) / sizeof(bufs[0])), 5)) != MLSTM_OK) return s;
    }
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // the workspace: the MFMA part's own, then the padded copies, then the state
    // handed from the MFMA part to the tail
    char* pad_base = (char*)workspace + align256(pl.main_bytes);
    float* C_mid = nullptr; float* n_mid = nullptr; float* m_mid = nullptr;
    if (pl.mid_bytes > 0) {
        char* base = pad_base + pl.pad_bytes;
        C_mid = (float*)base;
        n_mid = (float*)(base + align256(heads * d_v * d_qk * 4));
        m_mid = (float*)(base + align256(heads * d_v * d_qk * 4) + align256(heads * d_qk * 4));
    }
    if (pl.S_main > 0) {
        mlstm::FwdArgs a = make_fwd_args(B, NH, pl.S_main, pl.dq_run, d_v, chunk, dtype);
        a.Sx = S;
        a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre; a.h = h_out;
        float* C_dst = pl.tail ? C_mid : C_final;
        float* n_dst = pl.tail ? n_mid : n_final;
        a.C = C_dst; a.n = n_dst; a.m = pl.tail ? m_mid : m_final;
        a.C0 = C_init; a.n0 = n_init; a.m0 = m_init;
        a.ws = workspace; a.ws_bytes = pl.main_bytes; a.stream = st;
        if (ep) {
            a.ep_x = ep->x; a.ep_z = ep->z; a.ep_gw = ep->gw; a.ep_gb = ep->gb; a.ep_sw = ep->sw;
            a.ep_eps = ep->eps; a.ep_act = ep->act;
        }
        if (pl.pad) {
            // zero-padded copies (whole sequences, so the token stride stays S); the
            // staged entry points take no initial state, so C'_0 and n'_0 only come
            // with both stages
            char* p = pad_base;
            void* q_p = p; p += pl.qk_bytes;
            void* k_p = p; p += pl.qk_bytes;
            float* C0_p = (float*)p; p += pl.cpad_bytes;
            float* n0_p = (float*)p; p += pl.npad_bytes;
            float* C_p = (float*)p; p += pl.cpad_bytes;
            float* n_p = (float*)p;
            const size_t el = 2, rows = heads * (size_t)S;
            if (stages & 1) {
                e = mlstm::launch_copy_cols(q, q_p, rows, (size_t)d_qk * el, (size_t)pl.dq_run * el, st);
                if (e == hipSuccess) e = mlstm::launch_copy_cols(k, k_p, rows, (size_t)d_qk * el, (size_t)pl.dq_run * el, st);
                if (e == hipSuccess && given == 3)
                    e = mlstm::launch_copy_cols(C_init, C0_p, heads * d_v, (size_t)d_qk * 4, (size_t)pl.dq_run * 4, st);
                if (e == hipSuccess && given == 3)
                    e = mlstm::launch_copy_cols(n_init, n0_p, heads, (size_t)d_qk * 4, (size_t)pl.dq_run * 4, st);
            }
            a.q = q_p; a.k = k_p;
            if (given == 3) { a.C0 = C0_p; a.n0 = n0_p; }
            a.C = C_p; a.n = n_p;
            if (e == hipSuccess && (stages & 1)) e = mlstm::launch_fwd_mfma_prepare(a);
            if (e == hipSuccess && (stages & 2)) e = mlstm::launch_fwd_mfma_scan(a);
            if (e == hipSuccess && (stages & 2))
                e = mlstm::launch_copy_cols(C_p, C_dst, heads * d_v, (size_t)pl.dq_run * 4, (size_t)d_qk * 4, st);
            if (e == hipSuccess && (stages & 2))
                e = mlstm::launch_copy_cols(n_p, n_dst, heads, (size_t)pl.dq_run * 4, (size_t)d_qk * 4, st);
        } else {
            if (stages & 1) e = mlstm::launch_fwd_mfma_prepare(a);
            if (e == hipSuccess && (stages & 2)) e = mlstm::launch_fwd_mfma_scan(a);
        }
    }
    if (e == hipSuccess && pl.tail && (stages & 2)) {
        mlstm::FwdArgs a = make_fwd_args(B, NH, S, d_qk, d_v, chunk, dtype);
        a.t_begin = pl.S_main;
        a.q = q; a.k = k; a.v = v; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre; a.h = h_out;
        a.C = C_final; a.n = n_final; a.m = m_final;
        if (pl.S_main > 0) { a.C0 = C_mid; a.n0 = n_mid; a.m0 = m_mid; }
        else { a.C0 = C_init; a.n0 = n_init; a.m0 = m_init; }
        a.stream = st;
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
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr, nullptr,
                      h_out, C_final, n_final, m_final, workspace, workspace_bytes, stream, 3, false);
}

mlstm_status mlstm_fwd_parallel_state(const void* q, const void* k, const void* v,
                                      const float* i_pre, const float* f_pre, const float* o_pre,
                                      int B, int NH, int S, int d_qk, int d_v, int chunk,
                                      mlstm_dtype dtype,
                                      const float* C_init, const float* n_init, const float* m_init,
                                      void* h_out, float* C_final, float* n_final, float* m_final,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, C_init, n_init, m_init,
                      h_out, C_final, n_final, m_final, workspace, workspace_bytes, stream, 3, true);
}

// How a forward with the block epilogue runs: fused into the scan's output rows when
// the caller asks for it and the shape runs whole on the matrix cores with one value
// tile per head; otherwise the forward writes h into the workspace (after its own
// part) and the epilogue kernel reads it from there.
struct BlockPlan {
    bool fused;
    size_t fwd_bytes;       // the forward's own workspace
    size_t total;           // plus h when not fused
};

static BlockPlan plan_block(int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype, int fuse) {
    BlockPlan bp = {};
    const FwdPlan pl = plan_fwd(B, NH, S, d_qk, d_v, chunk, dtype);
    if (fuse && dtype == MLSTM_BF16 && pl.S_main == S && !pl.tail)
        bp.fused = mlstm::mfma_fwd_block_fusable(make_fwd_args(B, NH, S, pl.dq_run, d_v, chunk, dtype));
    bp.fwd_bytes = pl.total();
    const size_t el = dtype == MLSTM_BF16 ? 2 : 4;
    bp.total = bp.fused ? bp.fwd_bytes : align256(bp.fwd_bytes) + align256((size_t)B * NH * S * d_v * el);
    return bp;
}

size_t mlstm_fwd_block_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                                       int fuse) {
    if (check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype, false) != MLSTM_OK) return 0;
    return plan_block(B, NH, S, d_qk, d_v, chunk, dtype, fuse).total;
}

mlstm_status mlstm_fwd_parallel_block(const void* q, const void* k, const void* v,
                                      const float* i_pre, const float* f_pre, const float* o_pre,
                                      const void* x, const void* z,
                                      const float* gn_weight, const float* gn_bias, const float* skip_weight,
                                      int B, int NH, int S, int d_qk, int d_v, int chunk,
                                      float eps, mlstm_gate_act act, mlstm_dtype dtype, int fuse,
                                      void* y_out, float* C_final, float* n_final, float* m_final,
                                      void* workspace, size_t workspace_bytes, void* stream) {
    mlstm_status s = check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype, false);
    if (fuse != 0 && fuse != 1) return fail(MLSTM_ERR_INVALID_ARG, "fuse=%d is neither 0 nor 1", fuse);
    if (s != MLSTM_OK) return s;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(MLSTM_ERR_INVALID_ARG, "eps=%g must be finite and >= 0", eps);
    if (act != MLSTM_GATE_SIGMOID && act != MLSTM_GATE_SWISH)
        return fail(MLSTM_ERR_INVALID_ARG, "act=%d is neither MLSTM_GATE_SIGMOID nor MLSTM_GATE_SWISH", (int)act);
    const void* eptrs[] = {x, z, gn_weight, gn_bias, skip_weight, y_out};
    const char* enames[] = {"x", "z", "gn_weight", "gn_bias", "skip_weight", "y_out"};
    for (int p = 0; p < 6; ++p) {
        if (!eptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", enames[p]);
        if (!aligned16(eptrs[p])) return fail(MLSTM_ERR_INVALID_ARG, "%s is not 16-byte aligned", enames[p]);
    }
    const BlockPlan bp = plan_block(B, NH, S, d_qk, d_v, chunk, dtype, fuse);
    if (bp.total > 0) {
        if (!workspace || workspace_bytes < bp.total)
            return fail(MLSTM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, bp.total);
        if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    }
    {
        // y is written while x and z are still read, and the parameters are read throughout
        const size_t el = dtype == MLSTM_BF16 ? 2 : 4;
        const size_t yb = (size_t)B * NH * S * d_v * el, pb = (size_t)NH * d_v * 4;
        const Buf bufs[] = {
            {y_out, yb, "y_out"},
            {x, yb, "x"}, {z, yb, "z"}, {gn_weight, pb, "gn_weight"}, {gn_bias, pb, "gn_bias"},
            {skip_weight, pb, "skip_weight"}, {bp.total > 0 ? workspace : nullptr, bp.total, "workspace"},
        };
        if ((s = check_disjoint(bufs, (int)(sizeof(bufs) / sizeof(bufs[0])), 1)) != MLSTM_OK) return s;
    }
    if (bp.fused) {
        const EpiIn e = {x, z, gn_weight, gn_bias, skip_weight, eps, (int)act};
        return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr,
                          nullptr, y_out, C_final, n_final, m_final, workspace, bp.fwd_bytes, stream, 3, false, &e);
    }
    void* h_tmp = (char*)workspace + align256(bp.fwd_bytes);
    s = fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr, nullptr,
                   h_tmp, C_final, n_final, m_final, workspace, bp.fwd_bytes, stream, 3, false);
    if (s != MLSTM_OK) return s;
    mlstm::EpilogueArgs a = {};
    a.h = h_tmp; a.x = x; a.z = z; a.gn_w = gn_weight; a.gn_b = gn_bias; a.skip_w = skip_weight;
    a.B = B; a.NH = NH; a.S = S; a.dv = d_v; a.eps = eps; a.act = (int)act; a.dtype = dtype; a.y = y_out;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = mlstm::launch_epilogue(a);
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t mlstm_fwd_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

mlstm_status mlstm_fwd_parallel_noalloc(const void* q, const void* k, const void* v,
                                        const float* i_pre, const float* f_pre, const float* o_pre,
                                        int B, int NH, int S, int d_qk, int d_v, int chunk,
                                        mlstm_dtype dtype,
                                        void* h_out, float* C_final, float* n_final, float* m_final,
                                        void* stream) {
    // sizes first: a call the scratch array cannot serve is rejected before any HIP call
    mlstm_status s = check_fwd_sizes(B, NH, S, d_qk, d_v, chunk, dtype, false);
    if (s != MLSTM_OK) return s;
    const size_t need = plan_fwd(B, NH, S, d_qk, d_v, chunk, dtype).total();
    if (need > NOALLOC_SCRATCH_BYTES)
        return fail(MLSTM_ERR_UNSUPPORTED,
                    "this forward needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                    "(use mlstm_fwd_parallel with a caller-provided workspace)",
                    need, NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (need > 0 && (s = scratch_for_current_device(&ws)) != MLSTM_OK) return s;
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr, nullptr,
                      h_out, C_final, n_final, m_final, ws, need > 0 ? NOALLOC_SCRATCH_BYTES : 0, stream, 3, false);
}

mlstm_status mlstm_fwd_prepare(const void* q, const void* k, const float* i_pre, const float* f_pre,
                               int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, nullptr, i_pre, f_pre, nullptr, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr,
                      nullptr, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes, stream, 1, false);
}

mlstm_status mlstm_fwd_scan(const void* q, const void* k, const void* v,
                            const float* i_pre, const float* f_pre, const float* o_pre,
                            int B, int NH, int S, int d_qk, int d_v, int chunk, mlstm_dtype dtype,
                            void* h_out, float* C_final, float* n_final, float* m_final,
                            void* workspace, size_t workspace_bytes, void* stream) {
    return fwd_common(q, k, v, i_pre, f_pre, o_pre, B, NH, S, d_qk, d_v, chunk, dtype, nullptr, nullptr, nullptr,
                      h_out, C_final, n_final, m_final, workspace, workspace_bytes, stream, 2, false);
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
    {
        // C, n and m are updated in place (each element read and written by one
        // thread) and h is written: none of them may share memory with anything else
        const size_t heads = (size_t)B * NH;
        const Buf bufs[] = {
            {C, heads * d_v * d_qk * 4, "C"}, {n, heads * d_qk * 4, "n"}, {m, heads * 4, "m"},
            {h_out, heads * d_v * el, "h_out"},
            {q, heads * d_qk * el, "q"}, {k, heads * d_qk * el, "k"}, {v, heads * d_v * el, "v"},
            {i_pre, heads * 4, "i_pre"}, {f_pre, heads * 4, "f_pre"}, {o_pre, heads * d_v * 4, "o_pre"},
        };
        if ((s = check_disjoint(bufs, (int)(sizeof(bufs) / sizeof(bufs[0])), 4)) != MLSTM_OK) return s;
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

// sizes the backward accepts: those of the forward without the chunk
static mlstm_status check_bwd_sizes(int B, int NH, int S, int dqk, int dv, mlstm_dtype dt) {
    mlstm_status s = check_fwd_sizes(B, NH, S, dqk, dv, 16, dt, true);
    if (s != MLSTM_OK) return s;
    if (S > 65535 * 64) return fail(MLSTM_ERR_UNSUPPORTED, "S=%d exceeds the backward's %d tokens", S, 65535 * 64);
    if ((long long)B * NH * ((S + 63) / 64) > 0x7fffffffLL)
        return fail(MLSTM_ERR_UNSUPPORTED, "B*NH*ceil(S/64) exceeds the backward's grid");
    return MLSTM_OK;
}

static mlstm::BwdArgs make_bwd_args(int B, int NH, int S, int dqk, int dv, mlstm_dtype dt) {
    mlstm::BwdArgs a = {};
    a.B = B; a.NH = NH; a.S = S; a.dqk = dqk; a.dv = dv; a.dtype = dt;
    return a;
}

size_t mlstm_bwd_workspace_bytes(int B, int NH, int S, int d_qk, int d_v, mlstm_dtype dtype) {
    if (check_bwd_sizes(B, NH, S, d_qk, d_v, dtype) != MLSTM_OK) return 0;
    return mlstm::bwd_workspace_bytes(make_bwd_args(B, NH, S, d_qk, d_v, dtype));
}

mlstm_status mlstm_bwd_parallel(const void* q, const void* k, const void* v,
                                const float* i_pre, const float* f_pre, const float* o_pre,
                                const void* dh,
                                int B, int NH, int S, int d_qk, int d_v, mlstm_dtype dtype,
                                float* grad_q, float* grad_k, float* grad_v,
                                float* grad_i, float* grad_f, float* grad_o,
                                void* workspace, size_t workspace_bytes, void* stream) {
    mlstm_status s = check_bwd_sizes(B, NH, S, d_qk, d_v, dtype);
    if (s != MLSTM_OK) return s;
    const void* ptrs[] = {q, k, v, i_pre, f_pre, o_pre, dh, grad_q, grad_k, grad_v, grad_i, grad_f, grad_o};
    const char* names[] = {"q", "k", "v", "i_pre", "f_pre", "o_pre", "dh",
                           "grad_q", "grad_k", "grad_v", "grad_i", "grad_f", "grad_o"};
    const unsigned align[] = {16, 16, 16, 4, 4, 16, 16, 16, 16, 16, 4, 4, 16};
    for (int p = 0; p < 13; ++p) {
        if (!ptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", names[p]);
        if (!aligned(ptrs[p], align[p]))
            return fail(MLSTM_ERR_INVALID_ARG, "%s is not %u-byte aligned", names[p], align[p]);
    }
    mlstm::BwdArgs a = make_bwd_args(B, NH, S, d_qk, d_v, dtype);
    const size_t need = mlstm::bwd_workspace_bytes(a);
    if (!workspace || workspace_bytes < need)
        return fail(MLSTM_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(MLSTM_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    a.q = q; a.k = k; a.v = v; a.dh = dh; a.i_pre = i_pre; a.f_pre = f_pre; a.o_pre = o_pre;
    a.dq = grad_q; a.dk = grad_k; a.dvv = grad_v; a.di = grad_i; a.df = grad_f; a.dout = grad_o;
    a.ws = workspace;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = mlstm::launch_bwd(a);
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mlstm_status mlstm_block_epilogue(const void* h, const void* x, const void* z,
                                  const float* gn_weight, const float* gn_bias, const float* skip_weight,
                                  int B, int NH, int S, int d_v, float eps, mlstm_gate_act act,
                                  mlstm_dtype dtype, void* y_out, void* stream) {
    if (B < 1 || NH < 1 || S < 1)
        return fail(MLSTM_ERR_INVALID_ARG, "B=%d, NH=%d, S=%d must all be >= 1", B, NH, S);
    if (d_v < 16 || d_v > MAX_DIM || d_v % 16 != 0)
        return fail(MLSTM_ERR_INVALID_ARG, "d_v=%d must be a multiple of 16 in [16, %d]", d_v, MAX_DIM);
    mlstm_status s = check_dtype(dtype);
    if (s != MLSTM_OK) return s;
    if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(MLSTM_ERR_INVALID_ARG, "eps=%g must be finite and >= 0", eps);
    if (act != MLSTM_GATE_SIGMOID && act != MLSTM_GATE_SWISH)
        return fail(MLSTM_ERR_INVALID_ARG, "act=%d is neither MLSTM_GATE_SIGMOID nor MLSTM_GATE_SWISH", (int)act);
    if ((long long)B * NH * S * d_v > (1LL << 40) || (long long)B * NH * S > 0x7fffffffLL * 4)
        return fail(MLSTM_ERR_UNSUPPORTED, "tensor too large");
    const void* ptrs[] = {h, x, z, gn_weight, gn_bias, skip_weight, y_out};
    const char* names[] = {"h", "x", "z", "gn_weight", "gn_bias", "skip_weight", "y_out"};
    for (int p = 0; p < 7; ++p) {
        if (!ptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", names[p]);
        if (!aligned16(ptrs[p])) return fail(MLSTM_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[p]);
    }
    const size_t bytes = (size_t)B * NH * S * d_v * (dtype == MLSTM_BF16 ? 2 : 4);
    for (int p = 0; p < 3; ++p)
        if (ptrs[p] != y_out && overlaps(ptrs[p], bytes, y_out, bytes))
            return fail(MLSTM_ERR_INVALID_ARG, "y_out partly overlaps %s", names[p]);
    mlstm::EpilogueArgs a = {};
    a.h = h; a.x = x; a.z = z; a.gn_w = gn_weight; a.gn_b = gn_bias; a.skip_w = skip_weight;
    a.B = B; a.NH = NH; a.S = S; a.dv = d_v; a.eps = eps; a.act = (int)act; a.dtype = dtype; a.y = y_out;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = mlstm::launch_epilogue(a);
    if (e != hipSuccess) return fail(MLSTM_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

mlstm_status slstm_fwd(const float* x_pre, const void* R, int B, int NH, int S, int d_h,
                       mlstm_forget_act forget, mlstm_dtype dtype,
                       const float* c_init, const float* n_init, const float* m_init, const float* h_init,
                       void* h_out, float* c_final, float* n_final, float* m_final, float* h_final,
                       void* stream) {
    if (B < 1 || NH < 1 || S < 1)
        return fail(MLSTM_ERR_INVALID_ARG, "B=%d, NH=%d, S=%d must all be >= 1", B, NH, S);
    mlstm_status s = check_dtype(dtype);
    if (s != MLSTM_OK) return s;
    const int dmax = dtype == MLSTM_BF16 ? 192 : 128;
    if (d_h < 16 || d_h % 16 != 0 || d_h > dmax)
        return fail(MLSTM_ERR_INVALID_ARG, "d_h=%d must be a multiple of 16 in [16, %d] for this dtype", d_h, dmax);
    if (forget != MLSTM_FORGET_SIGMOID && forget != MLSTM_FORGET_EXP)
        return fail(MLSTM_ERR_INVALID_ARG, "forget=%d is neither MLSTM_FORGET_SIGMOID nor MLSTM_FORGET_EXP",
                    (int)forget);
    if ((long long)NH * ((B + 7) / 8) > 0x7fffffffLL || (long long)B * NH * S * 4 * d_h > (1LL << 40))
        return fail(MLSTM_ERR_UNSUPPORTED, "tensor too large");
    const unsigned el = dtype == MLSTM_BF16 ? 2u : 4u;
    const void* ptrs[] = {x_pre, R, h_out, c_final, n_final, m_final, h_final};
    const char* names[] = {"x_pre", "R", "h_out", "c_final", "n_final", "m_final", "h_final"};
    const unsigned align[] = {16, 16, el, 8, 8, 8, 8};
    for (int p = 0; p < 7; ++p) {
        if (!ptrs[p]) return fail(MLSTM_ERR_INVALID_ARG, "%s is NULL", names[p]);
        if (!aligned(ptrs[p], align[p]))
            return fail(MLSTM_ERR_INVALID_ARG, "%s is not %u-byte aligned", names[p], align[p]);
    }
    const int given = (c_init != nullptr) + (n_init != nullptr) + (m_init != nullptr) + (h_init != nullptr);
    if (given != 0 && given != 4)
        return fail(MLSTM_ERR_INVALID_ARG, "c_init, n_init, m_init and h_init must be given together (or all NULL)");
    const size_t sb = (size_t)B * NH * d_h * 4;
    const void* ins[] = {c_init, n_init, m_init, h_init};
    const void* outs[] = {c_final, n_final, m_final, h_final};
    for (int i = 0; i < 4; ++i) {
        if (given && !aligned(ins[i], 8)) return fail(MLSTM_ERR_INVALID_ARG, "initial state is not 8-byte aligned");
        for (int o = 0; o < 4; ++o) {
            if (o != i && overlaps(outs[i], sb, outs[o], sb))
                return fail(MLSTM_ERR_INVALID_ARG, "the final state buffers overlap each other");
            if (given && overlaps(ins[i], sb, outs[o], sb) && !(i == o && ins[i] == outs[o]))
                return fail(MLSTM_ERR_INVALID_ARG, "an initial state buffer overlaps a final one (other than in place)");
        }
    }
    const size_t hb = (size_t)B * NH * S * d_h * el;
    for (int i = 0; i < 4; ++i)
        if (overlaps(h_out, hb, outs[i], sb) || (given && overlaps(h_out, hb, ins[i], sb)))
            return fail(MLSTM_ERR_INVALID_ARG, "h_out overlaps a state buffer");
    mlstm::SlstmArgs a = {};
    a.x_pre = x_pre; a.R = R; a.B = B; a.NH = NH; a.S = S; a.dh = d_h;
    a.forget_exp = forget == MLSTM_FORGET_EXP ? 1 : 0; a.dtype = dtype;
    a.c0 = c_init; a.n0 = n_init; a.m0 = m_init; a.h0 = h_init;
    a.h = h_out; a.c = c_final; a.n = n_final; a.m = m_final; a.hlast = h_final;
    a.stream = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = mlstm::launch_slstm(a);
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
