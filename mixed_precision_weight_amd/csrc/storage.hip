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

// x_d[m][p] = x[m][d_p] for p < K - k, 0 up to Kd32. Thread p (grid x) finds d_p
// once and walks blockDim.y-strided tokens.
__global__ __launch_bounds__(256) void k_gather_dense(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                      const int32_t* __restrict__ idx, int32_t k, int64_t Kd32,
                                                      uint16_t* __restrict__ xd)
{
    const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (p >= Kd32)
        return;
    const int64_t Kd = K - k;
    const int64_t j = p < Kd ? p + weak_before_dense(idx, k, (int)p) : -1;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y)
        xd[m * Kd32 + p] = j >= 0 ? x[m * K + j] : (uint16_t)0;
}

// y[m][i] = fp16(y_in + sum_c w_weak[i][c] x[m][idx_c]), y_in = y[m][i] (fp16) or 0
__global__ __launch_bounds__(256) void k_weak_add(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                  const int32_t* __restrict__ idx, int32_t k,
                                                  const uint16_t* __restrict__ ww, int64_t N, int add,
                                                  uint16_t* __restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N)
        return;
    for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
        float acc = add ? h2f(y[m * N + i]) : 0.0f;
        for (int c = 0; c < k; c++) {
            int32_t j = idx[c];
            j = (j >= 0 && j < K) ? j : 0;
            acc = __builtin_fmaf(h2f(ww[i * k + c]), h2f(x[m * K + j]), acc);
        }
        y[m * N + i] = f2h(acc);
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
    const int64_t Kd32 = storage_dense_cols32(d.K, d.k);
    hipError_t e = hipSuccess;
    if (Kd32 > 0) {
        uint16_t* xd = static_cast<uint16_t*>(ws);
        const unsigned gy = (unsigned)(M < 64 ? M : 64);
        hipLaunchKernelGGL(k_gather_dense, dim3((unsigned)((Kd32 + 255) / 256), gy), dim3(256), 0, s, d.x, M, d.K,
                           d.idx, d.k, Kd32, xd);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        LinearDesc dd = d;  // the 3-bit codes against x_d as a layer of Kd32 columns, no weak columns
        dd.x = xd;
        dd.K = Kd32;
        dd.k = 0;
        dd.idx = nullptr;
        dd.ww = nullptr;
        e = launch_linear_any(dd, M, s);
        if (e != hipSuccess)
            return e;
    }
    if (d.k > 0 || Kd32 == 0) {
        const unsigned gy = (unsigned)(M < 256 ? M : 256);
        hipLaunchKernelGGL(k_weak_add, dim3((unsigned)((d.N + 255) / 256), gy), dim3(256), 0, s, d.x, M, d.K,
                           d.idx, d.k, d.ww, d.N, Kd32 > 0 ? 1 : 0, d.y);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace owq
