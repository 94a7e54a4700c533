// api.cpp -- the C ABI of libowq.so: synchronous argument validation, then
// kernel dispatch on the caller's stream. Declarations and the contract of
// every entry point are in include/owq.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/owq.h"
#include "owq_launch.h"

namespace {

thread_local char g_err[512] = "";

owq_status fail(owq_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

owq_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) {
        g_err[0] = '\0';
        return OWQ_OK;
    }
    return fail(OWQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr int64_t kMaxK = 65536;

owq_status check_k_dim(int64_t K)
{
    if (K < 32 || K > kMaxK || K % 32 != 0)
        return fail(OWQ_ERR_SHAPE, "K = %lld: need 32 <= K <= %lld and K %% 32 == 0", (long long)K,
                    (long long)kMaxK);
    return OWQ_OK;
}

bool check_enabled()
{
    static const bool on = [] {
        const char* e = getenv("OWQ_CHECK");
        return e && e[0] == '1';
    }();
    return on;
}

// Optional (OWQ_CHECK=1): synchronous copy of weak_idx and a host check that it
// is strictly ascending inside [0, K).
owq_status check_idx_on_host(const int32_t* idx, int32_t k, int64_t K, hipStream_t s)
{
    if (!check_enabled() || k == 0)
        return OWQ_OK;
    std::vector<int32_t> h((size_t)k);
    hipError_t e = hipMemcpyAsync(h.data(), idx, (size_t)k * sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess)
        e = hipStreamSynchronize(s);
    if (e != hipSuccess)
        return hip_status(e, "OWQ_CHECK copy of weak_idx");
    for (int32_t c = 0; c < k; c++) {
        if (h[c] < 0 || h[c] >= K || (c > 0 && h[c] <= h[c - 1]))
            return fail(OWQ_ERR_RANGE, "weak_idx[%d] = %d is not strictly ascending in [0, %lld)", c, h[c],
                        (long long)K);
    }
    return OWQ_OK;
}

owq_status check_layer(const owq_layer* L, int64_t M, const uint16_t* x, const uint16_t* y)
{
    if (!L)
        return fail(OWQ_ERR_NULL, "layer is NULL");
    if (L->bits != 3)
        return fail(OWQ_ERR_UNSUPPORTED, "bits = %d: only 3-bit codes are supported", L->bits);
    if (L->N < 1 || L->N > INT32_MAX)
        return fail(OWQ_ERR_SHAPE, "N = %lld out of range", (long long)L->N);
    owq_status st = check_k_dim(L->K);
    if (st != OWQ_OK)
        return st;
    if (M < 1 || M > INT32_MAX)
        return fail(OWQ_ERR_SHAPE, "M = %lld out of range", (long long)M);
    if (L->k < 0 || L->k > L->K)
        return fail(OWQ_ERR_RANGE, "k = %d outside [0, K = %lld]", L->k, (long long)L->K);
    if (!L->qcodes || !L->scales || !L->zeros || !x || !y)
        return fail(OWQ_ERR_NULL, "qcodes, scales, zeros, x and y must be non-NULL");
    if (L->k > 0 && (!L->weak_idx || !L->w_weak))
        return fail(OWQ_ERR_NULL, "weak_idx and w_weak must be non-NULL when k > 0");
    if (!aligned(x, 16) || !aligned(L->qcodes, 4) || !aligned(L->scales, 2) || !aligned(y, 2) ||
        (L->k > 0 && (!aligned(L->weak_idx, 4) || !aligned(L->w_weak, 2))))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (x: 16 B, qcodes/weak_idx: 4 B, fp16 arrays: 2 B)");
    return OWQ_OK;
}

owq::LinearDesc desc_of(const owq_layer* L, const uint16_t* x, uint16_t* y)
{
    owq::LinearDesc d;
    d.q = L->qcodes;
    d.s = L->scales;
    d.z = L->zeros;
    d.idx = L->k > 0 ? L->weak_idx : nullptr;
    d.ww = L->k > 0 ? L->w_weak : nullptr;
    d.x = x;
    d.y = y;
    d.N = L->N;
    d.K = L->K;
    d.k = L->k;
    return d;
}

}  // namespace

extern "C" {

const char* owq_status_string(owq_status s)
{
    switch (s) {
    case OWQ_OK: return "OWQ_OK";
    case OWQ_ERR_NULL: return "OWQ_ERR_NULL: a required pointer is NULL";
    case OWQ_ERR_SHAPE: return "OWQ_ERR_SHAPE: a dimension is out of range";
    case OWQ_ERR_RANGE: return "OWQ_ERR_RANGE: k or an index is out of range";
    case OWQ_ERR_ALIGN: return "OWQ_ERR_ALIGN: a device pointer is misaligned";
    case OWQ_ERR_UNSUPPORTED: return "OWQ_ERR_UNSUPPORTED: unsupported configuration";
    case OWQ_ERR_WORKSPACE: return "OWQ_ERR_WORKSPACE: workspace too small";
    case OWQ_ERR_HIP: return "OWQ_ERR_HIP: HIP runtime error";
    }
    return "unknown owq_status";
}

const char* owq_last_error(void) { return g_err; }

size_t owq_calibrate_workspace_bytes(int64_t N, int64_t K, int64_t T)
{
    if (N < 1 || T < 1 || K < 32 || K > kMaxK || K % 32 != 0 || N > INT32_MAX)
        return 0;
    return owq::calib_plan(N, K, T).total;
}

owq_status owq_calibrate_score(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                               double* lambda, double* score, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    if (!W || !X || !lambda || !score || !workspace)
        return fail(OWQ_ERR_NULL, "W, X, lambda, score and workspace must be non-NULL");
    if (N < 1 || N > INT32_MAX || T < 1)
        return fail(OWQ_ERR_SHAPE, "N = %lld, T = %lld: need N, T >= 1", (long long)N, (long long)T);
    owq_status st = check_k_dim(K);
    if (st != OWQ_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(lambda, 8) || !aligned(score, 8) ||
        !aligned(workspace, 256))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (W, X: 16 B, lambda/score: 8 B, workspace: 256 B)");
    owq::CalibPlan p = owq::calib_plan(N, K, T);
    if (workspace_bytes < p.total)
        return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, p.total);
    return hip_status(owq::launch_calibrate(W, N, K, X, T, lambda, score, workspace, p,
                                            (hipStream_t)stream),
                      "owq_calibrate_score launch");
}

owq_status owq_select_weak(const double* score, int64_t K, int32_t k, int32_t* weak_idx, void* stream)
{
    if (!score)
        return fail(OWQ_ERR_NULL, "score must be non-NULL");
    if (K < 1 || K > (int64_t)1 << 24)
        return fail(OWQ_ERR_SHAPE, "K = %lld: need 1 <= K <= 2^24", (long long)K);
    if (k < 0 || k > K)
        return fail(OWQ_ERR_RANGE, "k = %d outside [0, K = %lld]", k, (long long)K);
    if (k > 0 && !weak_idx)
        return fail(OWQ_ERR_NULL, "weak_idx must be non-NULL when k > 0");
    if (!aligned(score, 8) || (k > 0 && !aligned(weak_idx, 4)))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (score: 8 B, weak_idx: 4 B)");
    if (k == 0) {
        g_err[0] = '\0';
        return OWQ_OK;
    }
    return hip_status(owq::launch_select(score, K, k, weak_idx, (hipStream_t)stream),
                      "owq_select_weak launch");
}

owq_status owq_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                    uint32_t* qcodes, uint16_t* scales, uint8_t* zeros, uint16_t* w_weak, void* stream)
{
    if (!W || !qcodes || !scales || !zeros)
        return fail(OWQ_ERR_NULL, "W, qcodes, scales and zeros must be non-NULL");
    if (N < 1 || N > INT32_MAX)
        return fail(OWQ_ERR_SHAPE, "N = %lld out of range", (long long)N);
    owq_status st = check_k_dim(K);
    if (st != OWQ_OK)
        return st;
    if (k < 0 || k > K)
        return fail(OWQ_ERR_RANGE, "k = %d outside [0, K = %lld]", k, (long long)K);
    if (k > 0 && (!weak_idx || !w_weak))
        return fail(OWQ_ERR_NULL, "weak_idx and w_weak must be non-NULL when k > 0");
    if (!aligned(W, 16) || !aligned(qcodes, 4) || !aligned(scales, 2) ||
        (k > 0 && (!aligned(weak_idx, 4) || !aligned(w_weak, 2))))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (W: 16 B, qcodes/weak_idx: 4 B, fp16: 2 B)");
    st = check_idx_on_host(weak_idx, k, K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    return hip_status(owq::launch_pack(W, N, K, k > 0 ? weak_idx : nullptr, k, qcodes, scales, zeros,
                                       k > 0 ? w_weak : nullptr, (hipStream_t)stream),
                      "owq_pack launch");
}

owq_status owq_linear(const owq_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* stream)
{
    owq_status st = check_layer(L, M, x, y);
    if (st != OWQ_OK)
        return st;
    st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    hipStream_t s = (hipStream_t)stream;
    owq::LinearDesc d = desc_of(L, x, y);
    if (M >= owq::gemm_min_m())
        return hip_status(owq::launch_gemm(d, M, s), "owq_linear (matrix-core) launch");
    // decode kernels, in token slices of the chosen kernel's capacity
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess;) {
        const bool mat = owq::decode_on_matrix_cores(M - m0);
        const int64_t cap = mat ? owq::kMfvMaxM : owq::gemv_max_tokens(L->K);
        const int64_t mm = M - m0 < cap ? M - m0 : cap;
        owq::LinearDesc dm = d;
        dm.x = x + m0 * L->K;
        dm.y = y + m0 * L->N;
        e = mat ? owq::launch_mfv(&dm, 1, (int)mm, s) : owq::launch_gemv(&dm, 1, (int)mm, s);
        m0 += mm;
    }
    return hip_status(e, "owq_linear (decode) launch");
}

owq_status owq_linear_batched(const owq_layer* Ls, const uint16_t* const* xs, uint16_t* const* ys,
                              int32_t count, int64_t M, void* stream)
{
    if (!Ls || !xs || !ys)
        return fail(OWQ_ERR_NULL, "Ls, xs and ys must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    if (M < 1 || M > owq::kMfvMaxM)
        return fail(OWQ_ERR_UNSUPPORTED, "M = %lld: the batched decode launch needs 1 <= M <= %d",
                    (long long)M, owq::kMfvMaxM);
    const bool mat = owq::decode_on_matrix_cores(M);
    std::vector<owq::LinearDesc> d((size_t)count);
    for (int32_t l = 0; l < count; l++) {
        owq_status st = check_layer(&Ls[l], M, xs[l], ys[l]);
        if (st != OWQ_OK)
            return fail(st, "layer %d: %s", l, g_err);
        st = check_idx_on_host(Ls[l].weak_idx, Ls[l].k, Ls[l].K, (hipStream_t)stream);
        if (st != OWQ_OK)
            return st;
        if (mat ? !owq::mfv_fits(M, Ls[l].K) : !owq::gemv_fits(M, Ls[l].K))
            return fail(OWQ_ERR_UNSUPPORTED, "layer %d: M = %lld, K = %lld outside the batched decode limits", l,
                        (long long)M, (long long)Ls[l].K);
        d[l] = desc_of(&Ls[l], xs[l], ys[l]);
    }
    hipError_t e = hipSuccess;
    for (int32_t l0 = 0; l0 < count && e == hipSuccess; l0 += owq::kGemvMaxLayers) {
        int n = count - l0 < owq::kGemvMaxLayers ? count - l0 : owq::kGemvMaxLayers;
        e = mat ? owq::launch_mfv(d.data() + l0, n, (int)M, (hipStream_t)stream)
                : owq::launch_gemv(d.data() + l0, n, (int)M, (hipStream_t)stream);
    }
    return hip_status(e, "owq_linear_batched launch");
}

int64_t owq_stream_read_sink_words(int64_t bytes) { return bytes > 0 ? owq::stream_read_sink_words(bytes) : 0; }

owq_status owq_stream_read(const void* src, int64_t bytes, uint32_t* sink, int64_t sink_words, void* stream)
{
    if (!src || !sink)
        return fail(OWQ_ERR_NULL, "src and sink must be non-NULL");
    if (bytes < 12 || bytes % 12 != 0 || bytes > ((int64_t)1 << 40))
        return fail(OWQ_ERR_SHAPE, "bytes = %lld: need 12 <= bytes <= 2^40 and bytes %% 12 == 0", (long long)bytes);
    if (!aligned(src, 4) || !aligned(sink, 4))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (src and sink: 4 B)");
    if (sink_words < owq::stream_read_sink_words(bytes))
        return fail(OWQ_ERR_RANGE, "sink_words = %lld: need %lld", (long long)sink_words,
                    (long long)owq::stream_read_sink_words(bytes));
    return hip_status(owq::launch_stream_read(src, bytes, sink, (hipStream_t)stream), "owq_stream_read launch");
}

}  // extern "C"
