// storage.hip -- the storage-favoured OWQ form (gfx950): only the dense columns'
// 3-bit codes are kept, the zero-filled weak columns are removed, next to the
// fp16 weak columns ([PL] "Storage Methods", paper appendix section 2 pp.10-11:
// the zeros are dropped, at the price of extra work in the product; [PL] =
// paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for Efficient
// Fine-Tuning and Inference of Large Language Models").
//
// Layout: row i holds the codes of its dense columns in ascending column order,
// 32 to a group (the latency form's slot layout), the last group filled with the
// zero point: qcodes [N][ceil((K - k) / 32)][3]. Steps, zero points and the weak
// block are the latency-favoured pack's (fit over the dense columns).
//
// The product is the extra work the pages mention: the activations at the dense
// columns are gathered into a workspace (x_d [M][Kd32], zero beyond K - k), the
// latency form's kernels multiply the 3-bit codes with x_d as a layer of Kd32
// columns and no weak columns, and a last kernel adds the weak columns' fp16
// product to y. The p-th dense column is d_p = p + #{c : idx_c - c <= p} for the
// ascending weak indices (idx_c - c counts the dense columns before idx_c and
// does not decrease with c), found by binary search.
//
// Built with -ffp-contract=off: the quantiser steps are single IEEE operations.
#include <algorithm>
#include <vector>

#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kSlotS[32] = {1,  6,  2,  7,  3,  8,  4,  9,  5,  10, 11, 16, 12, 17, 13, 18,
                            14, 19, 15, 20, 21, 26, 22, 27, 23, 28, 24, 29, 25, 30, 0,  31};

// #{c < k : idx[c] - c <= p}, idx ascending
__device__ __forceinline__ int weak_before_dense(const int32_t* __restrict__ idx, int k, int p)
{
    int lo = 0, hi = k;  // answer in [lo, hi]
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] - mid <= p)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// One 256-thread block per row (grid-stride): the row's dense min/max (weak
// entries zeroed, as in the latency pack), then thread t packs output groups
// t, t + 256, ...: the group's first dense column by binary search, the next
// ones by skipping weak columns in the LDS mask.
__global__ __launch_bounds__(256) void k_pack_storage(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                      const int32_t* __restrict__ idx, int32_t k,
                                                      uint32_t* __restrict__ q, uint16_t* __restrict__ scales,
                                                      uint8_t* __restrict__ zeros, uint16_t* __restrict__ ww)
{
    extern __shared__ uint32_t wmask[];  // [G] weak-column bit mask per 32-column group
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t G = K / 32;
    const int64_t Kd = K - k, Gd = (Kd + 31) / 32;

    for (int64_t g = tid; g < G; g += 256)
        wmask[g] = 0;
    __syncthreads();
    for (int64_t c = tid; c < k; c += 256) {
        const int32_t j = idx[c];
        if (j >= 0 && j < K)  // indices outside [0, K) break the caller contract; never touch memory with them
            atomicOr(&wmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    auto is_weak = [&](int64_t j) { return (wmask[j >> 5] >> (j & 31)) & 1u; };

    for (int64_t row = blockIdx.x; row < N; row += gridDim.x) {
        const uint16_t* wr = W + row * K;
        float lo = 0.0f, hi = 0.0f;
        for (int64_t p = tid; p < K / 8; p += 256) {
            const uint4 v = *reinterpret_cast<const uint4*>(wr + p * 8);
            const uint32_t h[4] = {v.x, v.y, v.z, v.w};
            const uint32_t m = (wmask[p >> 2] >> ((p & 3) * 8)) & 0xffu;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float f = ((m >> i) & 1u) ? 0.0f : h2f((uint16_t)(h[i >> 1] >> (16 * (i & 1))));
                lo = fminf(lo, f);
                hi = fmaxf(hi, f);
            }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        if (lane == 0) {
            red[0][wave] = lo;
            red[1][wave] = hi;
        }
        __syncthreads();
        lo = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
        hi = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
        uint16_t s16;
        int z;
        qparams_from_range(lo, hi, s16, z);
        const RtnRow rr = make_rtn_row(h2f(s16), z);
        for (int64_t g = tid; g < Gd; g += 256) {
            const int p0 = (int)(g * 32);
            int64_t j = p0 + weak_before_dense(idx, k, p0);  // the first dense column of the group
            uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll 4
            for (int c = 0; c < 32; c++) {
                uint32_t cd = (uint32_t)z;
                if (p0 + c < Kd) {
                    while (is_weak(j))
                        j++;
                    cd = (uint32_t)rtn_code(h2f(wr[j]), rr);
                    j++;
                }
                const int pos = 3 * kSlotS[c], wd = pos >> 5, off = pos & 31;
                o[wd] |= cd << off;
                if (off > 29)
                    o[wd + 1] |= cd >> (32 - off);
            }
            uint32_t* dst = q + (row * Gd + g) * 3;
            dst[0] = o[0];
            dst[1] = o[1];
            dst[2] = o[2];
        }
        if (tid == 0) {
            scales[row] = s16;
            zeros[row] = (uint8_t)z;
        }
        for (int64_t c = tid; c < k; c += 256) {
            const int32_t jw = idx[c];
            ww[row * k + c] = (jw >= 0 && jw < K) ? wr[jw] : (uint16_t)0;
        }
        __syncthreads();  // red[] is reused by the next row
    }
}

// Several layers' gathers and weak additions in one launch each: blocks
// [b0[l], b0[l+1]) of grid x belong to layer l, grid y walks the tokens.
struct StorageStep {
    const uint16_t* x;
    const int32_t* idx;
    const uint16_t* ww;
    uint16_t* xd;  // gather: the layer's x_d
    uint16_t* y;   // weak addition: the layer's y
    int64_t K, Kd32, N;
    int32_t k, add;
};

struct StorageBatch {
    StorageStep L[kGemvMaxLayers];
    int32_t b0[kGemvMaxLayers + 1];
    int32_t count;
};

__device__ __forceinline__ int storage_layer_of(const StorageBatch& b)
{
    int l = 0;
    while (l + 1 < b.count && (int)blockIdx.x >= b.b0[l + 1])
        l++;
    return l;
}

__global__ __launch_bounds__(256) void k_gather_dense_batched(const StorageBatch b, int64_t M)
{
    const int l = storage_layer_of(b);
    const StorageStep& L = b.L[l];
    const int64_t p = (int64_t)(blockIdx.x - b.b0[l]) * 256 + threadIdx.x;
    if (p >= L.Kd32)
        return;
    const int64_t Kd = L.K - L.k;
    const int64_t j = p < Kd ? p + weak_before_dense(L.idx, L.k, (int)p) : -1;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y)
        L.xd[m * L.Kd32 + p] = j >= 0 ? L.x[m * L.K + j] : (uint16_t)0;
}

// y[m][i] = fp16(y_in + sum_c w_weak[i][c] x[m][idx_c]) (y_in = y[m][i] or 0): a
// wave per row (4 rows per block); lane l takes the weak columns l, l + 64, ...
// (the row's weights read contiguously), the lane sums are added by a fixed
// butterfly, then y_in.
__global__ __launch_bounds__(256) void k_weak_add_batched(const StorageBatch b, int64_t M)
{
    const int l = storage_layer_of(b);
    const StorageStep& L = b.L[l];
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)(blockIdx.x - b.b0[l]) * 4 + (threadIdx.x >> 6);
    if (i >= L.N)  // wave-uniform
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float acc = 0.0f;
        for (int c = lane; c < L.k; c += 64) {
            int32_t j = L.idx[c];
            j = (j >= 0 && j < L.K) ? j : 0;
            acc = __builtin_fmaf(h2f(L.ww[i * L.k + c]), h2f(L.x[m * L.K + j]), acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) {
            const float yin = L.add ? h2f(L.y[m * L.N + i]) : 0.0f;
            L.y[m * L.N + i] = f2h(yin + acc);
        }
    }
}

}  // namespace

int64_t storage_dense_cols32(int64_t K, int32_t k) { return ((K - k + 31) / 32) * 32; }

size_t storage_workspace_bytes(int64_t K, int32_t k, int64_t M)
{
    const size_t b = (size_t)M * (size_t)storage_dense_cols32(K, k) * sizeof(uint16_t);
    return ((b + 255) & ~(size_t)255) + 256;
}

hipError_t launch_pack_storage(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                               uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s)
{
    const unsigned grid = (unsigned)(N < 4096 ? N : 4096);
    hipLaunchKernelGGL(k_pack_storage, dim3(grid), dim3(256), (size_t)(K / 32) * sizeof(uint32_t), s, W, N, K,
                       idx, k, q, scales, zeros, ww);
    return hipGetLastError();
}

hipError_t launch_linear_storage(const LinearDesc& d, int64_t M, void* ws, hipStream_t s)
{
    return launch_linear_storage_batched(&d, 1, M, &ws, s);
}

hipError_t launch_linear_storage_batched(const LinearDesc* d, int count, int64_t M, void* const* ws, hipStream_t s)
{
    for (int l0 = 0; l0 < count; l0 += kGemvMaxLayers) {
        const int n = std::min(count - l0, kGemvMaxLayers);
        const LinearDesc* dl = d + l0;
        // 1. x at the dense columns of every layer
        StorageBatch g{};
        std::vector<LinearDesc> dense;
        for (int i = 0; i < n; i++) {
            const int64_t Kd32 = storage_dense_cols32(dl[i].K, dl[i].k);
            if (Kd32 == 0)
                continue;
            StorageStep& L = g.L[g.count];
            L = StorageStep{dl[i].x, dl[i].idx, nullptr, static_cast<uint16_t*>(ws[l0 + i]), nullptr, dl[i].K, Kd32,
                            0, dl[i].k, 0};
            g.b0[0] = 0;
            g.b0[g.count + 1] = g.b0[g.count] + (int32_t)((Kd32 + 255) / 256);
            g.count++;
            LinearDesc dd = dl[i];  // the codes against x_d as a layer of Kd32 columns, no weak columns
            dd.x = L.xd;
            dd.K = Kd32;
            dd.k = 0;
            dd.idx = nullptr;
            dd.ww = nullptr;
            dense.push_back(dd);
        }
        hipError_t e = hipSuccess;
        bool fused = false;  // the weak columns went with the dense products
        if (g.count > 0) {
            hipLaunchKernelGGL(k_gather_dense_batched, dim3((unsigned)g.b0[g.count], (unsigned)std::min<int64_t>(M, 64)),
                               dim3(256), 0, s, g, M);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
            // 2. the dense products, in one decode launch when every layer fits it
            bool one = M <= kMfvMaxM && M < gemm_min_m();  // the kernels owq_linear_storage would use
            const bool mat = decode_on_matrix_cores(M);
            for (const LinearDesc& dd : dense)
                one = one && (mat ? mfv_fits(M, dd.K) : gemv_fits(M, dd.K));
            fused = one && !mat;
            if (fused) {
                // the vector-ALU decode adds the weak columns itself, gathered from the
                // full x at the original indices: one fp32 sum and one fp16 rounding
                int j = 0;
                for (int i = 0; i < n; i++) {
                    if (storage_dense_cols32(dl[i].K, dl[i].k) == 0)
                        continue;
                    LinearDesc& dd = dense[j++];
                    dd.k = dl[i].k;
                    dd.idx = dl[i].idx;
                    dd.ww = dl[i].ww;
                    dd.xw = dl[i].x;
                    dd.kw = dl[i].K;
                }
            }
            if (one) {
                e = mat ? launch_mfv(dense.data(), (int)dense.size(), (int)M, s)
                        : launch_gemv(dense.data(), (int)dense.size(), (int)M, s);
            } else {
                for (const LinearDesc& dd : dense)
                    if (e == hipSuccess)
                        e = launch_linear_any(dd, M, s);
            }
            if (e != hipSuccess)
                return e;
        }
        // 3. the weak columns of every layer (a layer with no dense columns gets
        // its whole product here)
        StorageBatch w{};
        for (int i = 0; i < n; i++) {
            const int64_t Kd32 = storage_dense_cols32(dl[i].K, dl[i].k);
            if ((dl[i].k == 0 || fused) && Kd32 > 0)
                continue;
            StorageStep& L = w.L[w.count];
            L = StorageStep{dl[i].x, dl[i].idx, dl[i].ww, nullptr, dl[i].y, dl[i].K, Kd32, dl[i].N, dl[i].k,
                            Kd32 > 0 ? 1 : 0};
            w.b0[0] = 0;
            w.b0[w.count + 1] = w.b0[w.count] + (int32_t)((dl[i].N + 3) / 4);
            w.count++;
        }
        if (w.count > 0) {
            hipLaunchKernelGGL(k_weak_add_batched, dim3((unsigned)w.b0[w.count], (unsigned)std::min<int64_t>(M, 256)),
                               dim3(256), 0, s, w, M);
            e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

}  // namespace owq
