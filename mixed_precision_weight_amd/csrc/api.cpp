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

// The last error again, prefixed with "<what> <i>: " (the message is copied
// first: formatting a buffer into itself is undefined).
owq_status fail_at(owq_status s, const char* what, int i)
{
    char msg[sizeof g_err];
    snprintf(msg, sizeof msg, "%s", g_err);
    return fail(s, "%s %d: %s", what, i, msg);
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

namespace owq {

hipError_t launch_linear_any(const LinearDesc& d, int64_t M, hipStream_t s)
{
    if (M >= gemm_min_m())
        return launch_gemm(d, M, s);
    // decode kernels, in token slices of the chosen kernel's capacity
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess;) {
        const bool mat = decode_on_matrix_cores(M - m0);
        const int64_t cap = mat ? kMfvMaxM : gemv_max_tokens(d.K);
        const int64_t mm = M - m0 < cap ? M - m0 : cap;
        LinearDesc dm = d;
        dm.x = d.x + m0 * d.K;
        dm.y = d.y + m0 * d.N;
        e = mat ? launch_mfv(&dm, 1, (int)mm, s) : launch_gemv(&dm, 1, (int)mm, s);
        m0 += mm;
    }
    return e;
}

}  // namespace owq

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

size_t owq_calibrate_batched_workspace_bytes(const owq_calib_item* items, int32_t count)
{
    if (!items || count < 1 || count > 64)
        return 0;
    size_t total = 0;
    for (int32_t l = 0; l < count; l++) {
        const size_t b = owq_calibrate_workspace_bytes(items[l].N, items[l].K, items[l].T);
        if (b == 0)
            return 0;
        total += (b + 255) & ~(size_t)255;
    }
    return total;
}

owq_status owq_calibrate_score_batched(const owq_calib_item* items, int32_t count, void* workspace,
                                       size_t workspace_bytes, void* stream)
{
    if (!items || !workspace)
        return fail(OWQ_ERR_NULL, "items and workspace must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    if (!aligned(workspace, 256))
        return fail(OWQ_ERR_ALIGN, "misaligned workspace (256 B)");
    std::vector<owq::CalibItem> it((size_t)count);
    std::vector<owq::CalibPlan> plans((size_t)count);
    std::vector<void*> ws((size_t)count);
    size_t off = 0;
    for (int32_t l = 0; l < count; l++) {
        const owq_calib_item& c = items[l];
        if (!c.W || !c.X || !c.lambda || !c.score)
            return fail(OWQ_ERR_NULL, "item %d: W, X, lambda and score must be non-NULL", l);
        if (c.N < 1 || c.N > INT32_MAX || c.T < 1)
            return fail(OWQ_ERR_SHAPE, "item %d: N = %lld, T = %lld: need N, T >= 1", l, (long long)c.N,
                        (long long)c.T);
        owq_status st = check_k_dim(c.K);
        if (st != OWQ_OK)
            return fail_at(st, "item", l);
        if (!aligned(c.W, 16) || !aligned(c.X, 16) || !aligned(c.lambda, 8) || !aligned(c.score, 8))
            return fail(OWQ_ERR_ALIGN, "item %d: misaligned pointer (W, X: 16 B, lambda/score: 8 B)", l);
        it[l] = owq::CalibItem{c.W, c.N, c.K, c.X, c.T, c.lambda, c.score};
        plans[l] = owq::calib_plan(c.N, c.K, c.T);
        ws[l] = static_cast<char*>(workspace) + off;
        off += (plans[l].total + 255) & ~(size_t)255;
    }
    if (workspace_bytes < off)
        return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, off);
    return hip_status(owq::launch_calibrate_batched(it.data(), count, ws.data(), plans.data(), (hipStream_t)stream),
                      "owq_calibrate_score_batched launch");
}

owq_status owq_calibrate_score_noalloc(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                                       double* lambda, double* score, void* stream)
{
    if (!W || !X || !lambda || !score)
        return fail(OWQ_ERR_NULL, "W, X, lambda and score must be non-NULL");
    if (N < 1 || N > INT32_MAX || T < 1)
        return fail(OWQ_ERR_SHAPE, "N = %lld, T = %lld: need N, T >= 1", (long long)N, (long long)T);
    owq_status st = check_k_dim(K);
    if (st != OWQ_OK)
        return st;
    if (!aligned(W, 16) || !aligned(X, 16) || !aligned(lambda, 8) || !aligned(score, 8))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (W, X: 16 B, lambda/score: 8 B)");
    owq::CalibPlan p = owq::calib_plan(N, K, T);
    if (p.total > owq::kCalibScratchBytes)
        return fail(OWQ_ERR_WORKSPACE,
                    "N = %lld, K = %lld, T = %lld need %zu bytes of workspace; the library's own holds %zu "
                    "(use owq_calibrate_score with a caller workspace)",
                    (long long)N, (long long)K, (long long)T, p.total, owq::kCalibScratchBytes);
    void* ws = nullptr;
    hipError_t e = owq::calib_scratch(&ws);
    if (e != hipSuccess)
        return hip_status(e, "owq_calibrate_score_noalloc: scratch lookup");
    return hip_status(owq::launch_calibrate(W, N, K, X, T, lambda, score, ws, p, (hipStream_t)stream),
                      "owq_calibrate_score_noalloc launch");
}

size_t owq_calibrate_noalloc_max_workspace(void) { return owq::kCalibScratchBytes; }

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

owq_status owq_select_weak_batched(const double* const* scores, const int64_t* Ks, const int32_t* ks,
                                   int32_t* const* weak_idxs, int32_t count, void* stream)
{
    if (!scores || !Ks || !ks || !weak_idxs)
        return fail(OWQ_ERR_NULL, "scores, Ks, ks and weak_idxs must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    for (int32_t i = 0; i < count; i++) {
        const int64_t K = Ks[i];
        const int32_t k = ks[i];
        if (!scores[i])
            return fail(OWQ_ERR_NULL, "selection %d: score must be non-NULL", i);
        if (K < 1 || K > (int64_t)1 << 24)
            return fail(OWQ_ERR_SHAPE, "selection %d: K = %lld: need 1 <= K <= 2^24", i, (long long)K);
        if (k < 0 || k > K)
            return fail(OWQ_ERR_RANGE, "selection %d: k = %d outside [0, K = %lld]", i, k, (long long)K);
        if (k > 0 && !weak_idxs[i])
            return fail(OWQ_ERR_NULL, "selection %d: weak_idx must be non-NULL when k > 0", i);
        if (!aligned(scores[i], 8) || (k > 0 && !aligned(weak_idxs[i], 4)))
            return fail(OWQ_ERR_ALIGN, "selection %d: misaligned pointer (score: 8 B, weak_idx: 4 B)", i);
    }
    return hip_status(owq::launch_select_batched(scores, Ks, ks, weak_idxs, count, (hipStream_t)stream),
                      "owq_select_weak_batched launch");
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

owq_status owq_pack_batched(const owq_pack_item* items, int32_t count, void* stream)
{
    if (!items)
        return fail(OWQ_ERR_NULL, "items must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    std::vector<owq::PackItem> it((size_t)count);
    for (int32_t l = 0; l < count; l++) {
        const owq_pack_item& c = items[l];
        if (!c.W || !c.qcodes || !c.scales || !c.zeros)
            return fail(OWQ_ERR_NULL, "item %d: W, qcodes, scales and zeros must be non-NULL", l);
        if (c.N < 1 || c.N > INT32_MAX)
            return fail(OWQ_ERR_SHAPE, "item %d: N = %lld out of range", l, (long long)c.N);
        owq_status st = check_k_dim(c.K);
        if (st != OWQ_OK)
            return fail_at(st, "item", l);
        if (c.k < 0 || c.k > c.K)
            return fail(OWQ_ERR_RANGE, "item %d: k = %d outside [0, K = %lld]", l, c.k, (long long)c.K);
        if (c.k > 0 && (!c.weak_idx || !c.w_weak))
            return fail(OWQ_ERR_NULL, "item %d: weak_idx and w_weak must be non-NULL when k > 0", l);
        if (!aligned(c.W, 16) || !aligned(c.qcodes, 4) || !aligned(c.scales, 2) ||
            (c.k > 0 && (!aligned(c.weak_idx, 4) || !aligned(c.w_weak, 2))))
            return fail(OWQ_ERR_ALIGN, "item %d: misaligned pointer (W: 16 B, qcodes/weak_idx: 4 B, fp16: 2 B)", l);
        st = check_idx_on_host(c.weak_idx, c.k, c.K, (hipStream_t)stream);
        if (st != OWQ_OK)
            return fail_at(st, "item", l);
        it[l] = owq::PackItem{c.W, c.N, c.K, c.k > 0 ? c.weak_idx : nullptr, c.k, c.qcodes, c.scales, c.zeros,
                              c.k > 0 ? c.w_weak : nullptr};
    }
    return hip_status(owq::launch_pack_batched(it.data(), count, (hipStream_t)stream), "owq_pack_batched launch");
}

owq_status owq_pack_search(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                           const double* lambda, uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                           uint16_t* w_weak, void* stream)
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
    if (!aligned(W, 16) || !aligned(qcodes, 4) || !aligned(scales, 2) || !aligned(lambda, 8) ||
        (k > 0 && (!aligned(weak_idx, 4) || !aligned(w_weak, 2))))
        return fail(OWQ_ERR_ALIGN,
                    "misaligned pointer (W: 16 B, lambda: 8 B, qcodes/weak_idx: 4 B, fp16: 2 B)");
    st = check_idx_on_host(weak_idx, k, K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    const int32_t* idx = k > 0 ? weak_idx : nullptr;
    hipError_t e = owq::launch_search(W, N, K, idx, k, lambda, scales, zeros, (hipStream_t)stream);
    if (e == hipSuccess)
        e = owq::launch_pack_given(W, N, K, idx, k, qcodes, scales, zeros, k > 0 ? w_weak : nullptr,
                                   (hipStream_t)stream);
    return hip_status(e, "owq_pack_search launch");
}

owq_status owq_pack_storage(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                            uint32_t* qcodes, uint16_t* scales, uint8_t* zeros, uint16_t* w_weak, void* stream)
{
    if (!W || !scales || !zeros || (!qcodes && k < K))
        return fail(OWQ_ERR_NULL, "W, scales, zeros and (unless k == K) qcodes must be non-NULL");
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
    return hip_status(owq::launch_pack_storage(W, N, K, k > 0 ? weak_idx : nullptr, k, qcodes, scales, zeros,
                                               k > 0 ? w_weak : nullptr, (hipStream_t)stream),
                      "owq_pack_storage launch");
}

size_t owq_linear_storage_workspace_bytes(int64_t K, int32_t k, int64_t M)
{
    if (K < 32 || K > kMaxK || K % 32 != 0 || k < 0 || k > K || M < 1 || M > INT32_MAX)
        return 0;
    return owq::storage_workspace_bytes(K, k, M);
}

owq_status owq_linear_storage(const owq_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    if (!L)
        return fail(OWQ_ERR_NULL, "layer is NULL");
    if (L->k == L->K && L->K >= 32 && !L->qcodes) {  // every column weak: no codes are stored
        owq_layer tmp = *L;
        tmp.qcodes = reinterpret_cast<const uint32_t*>(L->scales);
        return owq_linear_storage(&tmp, x, M, y, workspace, workspace_bytes, stream);
    }
    owq_status st = check_layer(L, M, x, y);
    if (st != OWQ_OK)
        return st;
    if (!workspace)
        return fail(OWQ_ERR_NULL, "workspace must be non-NULL");
    if (!aligned(workspace, 256))
        return fail(OWQ_ERR_ALIGN, "misaligned workspace (256 B)");
    const size_t need = owq::storage_workspace_bytes(L->K, L->k, M);
    if (workspace_bytes < need)
        return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
    st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    return hip_status(owq::launch_linear_storage(desc_of(L, x, y), M, workspace, (hipStream_t)stream),
                      "owq_linear_storage launch");
}

size_t owq_linear_storage_batched_workspace_bytes(const owq_layer* Ls, int32_t count, int64_t M)
{
    if (!Ls || count < 1 || count > 64)
        return 0;
    size_t total = 0;
    for (int32_t l = 0; l < count; l++) {
        const size_t b = owq_linear_storage_workspace_bytes(Ls[l].K, Ls[l].k, M);
        if (b == 0)
            return 0;
        total += (b + 255) & ~(size_t)255;
    }
    return total;
}

owq_status owq_linear_storage_batched(const owq_layer* Ls, const uint16_t* const* xs, uint16_t* const* ys,
                                      int32_t count, int64_t M, void* workspace, size_t workspace_bytes,
                                      void* stream)
{
    if (!Ls || !xs || !ys)
        return fail(OWQ_ERR_NULL, "Ls, xs and ys must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    if (!workspace)
        return fail(OWQ_ERR_NULL, "workspace must be non-NULL");
    if (!aligned(workspace, 256))
        return fail(OWQ_ERR_ALIGN, "misaligned workspace (256 B)");
    std::vector<owq::LinearDesc> d((size_t)count);
    std::vector<void*> ws((size_t)count);
    size_t off = 0;
    for (int32_t l = 0; l < count; l++) {
        owq_layer L = Ls[l];
        if (L.k == L.K && L.K >= 32 && !L.qcodes)  // every column weak: no codes are stored
            L.qcodes = reinterpret_cast<const uint32_t*>(L.scales);
        owq_status st = check_layer(&L, M, xs[l], ys[l]);
        if (st != OWQ_OK)
            return fail_at(st, "layer", l);
        st = check_idx_on_host(L.weak_idx, L.k, L.K, (hipStream_t)stream);
        if (st != OWQ_OK)
            return fail_at(st, "layer", l);
        d[l] = desc_of(&L, xs[l], ys[l]);
        ws[l] = static_cast<char*>(workspace) + off;
        off += (owq::storage_workspace_bytes(L.K, L.k, M) + 255) & ~(size_t)255;
    }
    if (workspace_bytes < off)
        return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, off);
    return hip_status(owq::launch_linear_storage_batched(d.data(), count, M, ws.data(), (hipStream_t)stream),
                      "owq_linear_storage_batched launch");
}

size_t owq_pack_optq_workspace_bytes(int64_t N, int64_t K, int32_t k)
{
    if (N < 1 || N > INT32_MAX || K < 32 || K > kMaxK || K % 32 != 0 || k < 0 || k > K)
        return 0;
    return owq::optq_plan(N, K, k).total;
}

owq_status owq_pack_optq(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                         const int32_t* weak_idx, int32_t k, uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                         uint16_t* w_weak, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!W || !X || !qcodes || !scales || !zeros || !workspace)
        return fail(OWQ_ERR_NULL, "W, X, qcodes, scales, zeros and workspace must be non-NULL");
    if (N < 1 || N > INT32_MAX || T < 1 || T > INT32_MAX)
        return fail(OWQ_ERR_SHAPE, "N = %lld, T = %lld out of range", (long long)N, (long long)T);
    owq_status st = check_k_dim(K);
    if (st != OWQ_OK)
        return st;
    if (k < 0 || k > K)
        return fail(OWQ_ERR_RANGE, "k = %d outside [0, K = %lld]", k, (long long)K);
    if (k > 0 && (!weak_idx || !w_weak))
        return fail(OWQ_ERR_NULL, "weak_idx and w_weak must be non-NULL when k > 0");
    if (!aligned(W, 16) || !aligned(X, 2) || !aligned(qcodes, 4) || !aligned(scales, 2) ||
        !aligned(workspace, 256) || (k > 0 && (!aligned(weak_idx, 4) || !aligned(w_weak, 2))))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (W: 16 B, workspace: 256 B, qcodes/weak_idx: 4 B, fp16: 2 B)");
    const owq::OptqPlan p = owq::optq_plan(N, K, k);
    if (workspace_bytes < p.total)
        return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, p.total);
    st = check_idx_on_host(weak_idx, k, K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    return hip_status(owq::launch_pack_optq(W, N, K, X, T, k > 0 ? weak_idx : nullptr, k, qcodes, scales, zeros,
                                            k > 0 ? w_weak : nullptr, workspace, p, (hipStream_t)stream),
                      "owq_pack_optq launch");
}

size_t owq_linear_backward_workspace_bytes(int64_t N, int64_t K, int32_t k)
{
    if (N < 1 || N > INT32_MAX || K < 32 || K > kMaxK || K % 32 != 0 || k < 0 || k > K)
        return 0;
    return owq::bwd_plan(N, K, k).total;
}

owq_status owq_linear_backward(const owq_layer* L, const uint16_t* x, const uint16_t* dy, int64_t M, uint16_t* dx,
                               float* dw_weak, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!L || !dy)
        return fail(OWQ_ERR_NULL, "layer and dy must be non-NULL");
    // check_layer wants an x and a y: x is read only for dw_weak, y is not used
    owq_status st = check_layer(L, M, x ? x : dy, dy);
    if (st != OWQ_OK)
        return st;
    if (dw_weak && L->k > 0 && !x)
        return fail(OWQ_ERR_NULL, "x must be non-NULL for dw_weak");
    if ((dx && !aligned(dx, 2)) || (dw_weak && !aligned(dw_weak, 4)) || !aligned(dy, 2))
        return fail(OWQ_ERR_ALIGN, "misaligned pointer (dy, dx: 2 B, dw_weak: 4 B)");
    owq::BwdPlan p = owq::bwd_plan(L->N, L->K, L->k);
    if (dx) {
        if (!workspace)
            return fail(OWQ_ERR_NULL, "workspace must be non-NULL when dx is requested");
        if (!aligned(workspace, 256))
            return fail(OWQ_ERR_ALIGN, "misaligned workspace (256 B)");
        if (workspace_bytes < p.total)
            return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, p.total);
    }
    st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    owq::LinearDesc d = desc_of(L, x, nullptr);
    return hip_status(owq::launch_linear_backward(d, dy, M, dx, dw_weak, workspace, p, (hipStream_t)stream),
                      "owq_linear_backward launch");
}

size_t owq_linear_backward_batched_workspace_bytes(const owq_layer* Ls, int32_t count)
{
    if (!Ls || count < 1 || count > 64)
        return 0;
    size_t total = 0;
    for (int32_t l = 0; l < count; l++) {
        const size_t b = owq_linear_backward_workspace_bytes(Ls[l].N, Ls[l].K, Ls[l].k);
        if (b == 0)
            return 0;
        total += (b + 255) & ~(size_t)255;
    }
    return total;
}

owq_status owq_linear_backward_batched(const owq_layer* Ls, const uint16_t* const* xs, const uint16_t* const* dys,
                                       int32_t count, int64_t M, uint16_t* const* dxs, float* const* dws,
                                       void* workspace, size_t workspace_bytes, void* stream)
{
    if (!Ls || !dys)
        return fail(OWQ_ERR_NULL, "Ls and dys must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    std::vector<owq::LinearDesc> d((size_t)count);
    std::vector<owq::BwdPlan> plans((size_t)count);
    std::vector<const uint16_t*> dy((size_t)count);
    std::vector<uint16_t*> dx((size_t)count);
    std::vector<float*> dw((size_t)count);
    std::vector<void*> ws((size_t)count);
    size_t need = 0;
    for (int32_t l = 0; l < count; l++) {
        const owq_layer* L = &Ls[l];
        const uint16_t* x = xs ? xs[l] : nullptr;
        dy[l] = dys[l];
        dx[l] = dxs ? dxs[l] : nullptr;
        dw[l] = dws ? dws[l] : nullptr;
        if (!dy[l])
            return fail(OWQ_ERR_NULL, "layer %d: dy must be non-NULL", l);
        owq_status st = check_layer(L, M, x ? x : dy[l], dy[l]);
        if (st != OWQ_OK)
            return fail_at(st, "layer", l);
        if (dw[l] && L->k > 0 && !x)
            return fail(OWQ_ERR_NULL, "layer %d: x must be non-NULL for dw_weak", l);
        if ((dx[l] && !aligned(dx[l], 2)) || (dw[l] && !aligned(dw[l], 4)) || !aligned(dy[l], 2))
            return fail(OWQ_ERR_ALIGN, "layer %d: misaligned pointer (dy, dx: 2 B, dw_weak: 4 B)", l);
        st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
        if (st != OWQ_OK)
            return st;
        d[l] = desc_of(L, x, nullptr);
        plans[l] = owq::bwd_plan(L->N, L->K, L->k);
        ws[l] = nullptr;
        if (dx[l]) {
            ws[l] = reinterpret_cast<void*>(need);  // offset for now
            need += (plans[l].total + 255) & ~(size_t)255;
        }
    }
    if (need > 0) {
        if (!workspace)
            return fail(OWQ_ERR_NULL, "workspace must be non-NULL when dx is requested");
        if (!aligned(workspace, 256))
            return fail(OWQ_ERR_ALIGN, "misaligned workspace (256 B)");
        if (workspace_bytes < need)
            return fail(OWQ_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, need);
        for (int32_t l = 0; l < count; l++)
            if (dx[l])
                ws[l] = static_cast<char*>(workspace) + reinterpret_cast<size_t>(ws[l]);
    }
    hipError_t e = hipSuccess;
    for (int32_t l0 = 0; l0 < count && e == hipSuccess; l0 += owq::kBwdMaxLayers) {
        const int n = count - l0 < owq::kBwdMaxLayers ? count - l0 : owq::kBwdMaxLayers;
        e = owq::launch_linear_backward_batched(d.data() + l0, dy.data() + l0, n, M, dx.data() + l0, dw.data() + l0,
                                                ws.data() + l0, plans.data() + l0, (hipStream_t)stream);
    }
    return hip_status(e, "owq_linear_backward_batched launch");
}

owq_status owq_pack_grouped(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                            int64_t G, uint32_t* qcodes, uint16_t* scales, uint8_t* zeros, uint16_t* w_weak,
                            void* stream)
{
    if (!W || !qcodes || !scales || !zeros)
        return fail(OWQ_ERR_NULL, "W, qcodes, scales and zeros must be non-NULL");
    if (N < 1 || N > INT32_MAX)
        return fail(OWQ_ERR_SHAPE, "N = %lld out of range", (long long)N);
    owq_status st = check_k_dim(K);
    if (st != OWQ_OK)
        return st;
    if (!owq::grouped_size_supported(G, K))
        return fail(OWQ_ERR_UNSUPPORTED, "G = %lld: need a power of two in [32, 2048] dividing K = %lld",
                    (long long)G, (long long)K);
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
    return hip_status(owq::launch_pack_grouped(W, N, K, k > 0 ? weak_idx : nullptr, k, G, qcodes, scales, zeros,
                                               k > 0 ? w_weak : nullptr, (hipStream_t)stream),
                      "owq_pack_grouped launch");
}

owq_status owq_linear_grouped(const owq_grouped_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* stream)
{
    if (!L)
        return fail(OWQ_ERR_NULL, "layer is NULL");
    owq_layer base{L->N, L->K, L->k, L->bits, L->qcodes, L->scales, L->zeros, L->weak_idx, L->w_weak};
    owq_status st = check_layer(&base, M, x, y);
    if (st != OWQ_OK)
        return st;
    if (!owq::grouped_size_supported(L->G, L->K))
        return fail(OWQ_ERR_UNSUPPORTED, "G = %lld: need a power of two in [32, 2048] dividing K = %lld",
                    (long long)L->G, (long long)L->K);
    st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    const owq::LinearDesc d = desc_of(&base, x, y);
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += owq::kGemvMaxM) {  // token slices
        const int64_t mm = M - m0 < owq::kGemvMaxM ? M - m0 : owq::kGemvMaxM;
        owq::LinearDesc dm = d;
        dm.x = d.x + m0 * d.K;
        dm.y = d.y + m0 * d.N;
        e = owq::launch_gemv_grouped(&dm, &L->G, 1, (int)mm, (hipStream_t)stream);
    }
    return hip_status(e, "owq_linear_grouped launch");
}

owq_status owq_linear_grouped_batched(const owq_grouped_layer* Ls, const uint16_t* const* xs, uint16_t* const* ys,
                                      int32_t count, int64_t M, void* stream)
{
    if (!Ls || !xs || !ys)
        return fail(OWQ_ERR_NULL, "Ls, xs and ys must be non-NULL");
    if (count < 1 || count > 64)
        return fail(OWQ_ERR_UNSUPPORTED, "count = %d: need 1 <= count <= 64", count);
    if (M < 1 || M > owq::kGemvMaxM)
        return fail(OWQ_ERR_UNSUPPORTED, "M = %lld: the batched group-wise launch needs 1 <= M <= %d",
                    (long long)M, owq::kGemvMaxM);
    std::vector<owq::LinearDesc> d((size_t)count);
    std::vector<int64_t> groups((size_t)count);
    for (int32_t l = 0; l < count; l++) {
        const owq_grouped_layer& g = Ls[l];
        owq_layer base{g.N, g.K, g.k, g.bits, g.qcodes, g.scales, g.zeros, g.weak_idx, g.w_weak};
        owq_status st = check_layer(&base, M, xs[l], ys[l]);
        if (st != OWQ_OK)
            return fail_at(st, "layer", l);
        if (!owq::grouped_size_supported(g.G, g.K))
            return fail(OWQ_ERR_UNSUPPORTED, "layer %d: G = %lld: need a power of two in [32, 2048] dividing K = %lld",
                        l, (long long)g.G, (long long)g.K);
        st = check_idx_on_host(g.weak_idx, g.k, g.K, (hipStream_t)stream);
        if (st != OWQ_OK)
            return st;
        d[l] = desc_of(&base, xs[l], ys[l]);
        groups[l] = g.G;
    }
    hipError_t e = hipSuccess;
    for (int32_t l0 = 0; l0 < count && e == hipSuccess; l0 += owq::kGemvMaxLayers) {
        const int n = count - l0 < owq::kGemvMaxLayers ? count - l0 : owq::kGemvMaxLayers;
        e = owq::launch_gemv_grouped(d.data() + l0, groups.data() + l0, n, (int)M, (hipStream_t)stream);
    }
    return hip_status(e, "owq_linear_grouped_batched launch");
}

owq_status owq_linear(const owq_layer* L, const uint16_t* x, int64_t M, uint16_t* y, void* stream)
{
    owq_status st = check_layer(L, M, x, y);
    if (st != OWQ_OK)
        return st;
    st = check_idx_on_host(L->weak_idx, L->k, L->K, (hipStream_t)stream);
    if (st != OWQ_OK)
        return st;
    return hip_status(owq::launch_linear_any(desc_of(L, x, y), M, (hipStream_t)stream), "owq_linear launch");
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
            return fail_at(st, "layer", l);
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
