// grouped.hip -- group-wise scales on top of OWQ (gfx950): the pack. The product
// runs in the decode kernel of gemv.hip (its group-wise mode).
//
// Every output row is split into groups of G consecutive input columns and each
// (row, group) gets its own step size and zero point, on top of the fp16 weak
// columns ([PL] "Comparison with group-wise quantization", paper p.8, which
// finds it adds little to OWQ; its grouped baseline uses G = 128; [PL] =
// paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for Efficient
// Fine-Tuning and Inference of Large Language Models"). Each (row, group) is
// fitted like a row of the per-row form on the group's dense columns; the weak
// columns take their group's zero point as code; the codes keep the per-row
// form's 32-per-3-words layout; steps and zero points are [N][K/G].
//
// Pack: one thread per 32-column code group. G / 32 consecutive lanes hold one
// (row, group); its min and max are a butterfly over those lanes. The weak
// entries are zeroed first (the fitted range always contains 0, so a zero
// changes neither end and gets the zero point as code), as in the per-row pack.
//
// Product (gemv.hip, group-wise mode of the decode kernel): each 32-column code
// group is decoded to exact (q - z) fp16 pairs with its own group's zero point,
// its 16 v_dot2 run from 0, and its group's step scales that partial sum into
// the row's fp32 accumulator (one rounding).
//
// Built with -ffp-contract=off: the quantiser steps are single IEEE operations.
#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kSlotG[32] = {1,  6,  2,  7,  3,  8,  4,  9,  5,  10, 11, 16, 12, 17, 13, 18,
                            14, 19, 15, 20, 21, 26, 22, 27, 23, 28, 24, 29, 25, 30, 0,  31};

template <int CG>
__global__ __launch_bounds__(256) void k_pack_grouped(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                      const int32_t* __restrict__ idx, int32_t k,
                                                      uint32_t* __restrict__ q, uint16_t* __restrict__ scales,
                                                      uint8_t* __restrict__ zeros)
{
    extern __shared__ uint32_t wmask[];  // [K / 32] weak-column bits per code group
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t NC = K / 32, NG = NC / CG;
    for (int64_t g = tid; g < NC; g += 256)
        wmask[g] = 0;
    __syncthreads();
    for (int64_t c = tid; c < k; c += 256) {
        const int32_t j = idx[c];
        if (j >= 0 && j < K)
            atomicOr(&wmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    const int64_t total = N * NC;
    const int64_t wave0 = ((int64_t)blockIdx.x * 256 + (tid & ~63));
    const int64_t stride = (int64_t)gridDim.x * 256;
    // every lane of a wave runs every iteration (the butterfly needs all of them)
    for (int64_t base = wave0; base < total; base += stride) {
        const int64_t t = base + lane;
        const bool valid = t < total;
        const int64_t tc = valid ? t : total - 1;
        const int64_t row = tc / NC, cg = tc % NC;
        uint32_t v[16];
        const uint4* p = reinterpret_cast<const uint4*>(W + row * K + cg * 32);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint4 w4 = p[i];
            v[4 * i + 0] = w4.x;
            v[4 * i + 1] = w4.y;
            v[4 * i + 2] = w4.z;
            v[4 * i + 3] = w4.w;
        }
        const uint32_t m = wmask[cg];
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; c++) {
            if ((m >> c) & 1u)
                v[c >> 1] &= (c & 1) ? 0x0000ffffu : 0xffff0000u;
            const float f = h2f((uint16_t)(v[c >> 1] >> (16 * (c & 1))));
            lo = fminf(lo, f);
            hi = fmaxf(hi, f);
        }
#pragma unroll
        for (int o = 1; o < CG; o <<= 1) {
            lo = fminf(lo, __shfl_xor(lo, o));
            hi = fmaxf(hi, __shfl_xor(hi, o));
        }
        uint16_t s16;
        int z;
        qparams_from_range(lo, hi, s16, z);
        const RtnRow rr = make_rtn_row(h2f(s16), z);
        uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 32; c++) {
            const uint32_t cd = (uint32_t)rtn_code(h2f((uint16_t)(v[c >> 1] >> (16 * (c & 1)))), rr);
            const int pos = 3 * kSlotG[c], wd = pos >> 5, off = pos & 31;
            o[wd] |= cd << off;
            if (off > 29)
                o[wd + 1] |= cd >> (32 - off);
        }
        if (valid) {
            uint32_t* dst = q + tc * 3;
            dst[0] = o[0];
            dst[1] = o[1];
            dst[2] = o[2];
            if (cg % CG == 0) {
                scales[row * NG + cg / CG] = s16;
                zeros[row * NG + cg / CG] = (uint8_t)z;
            }
        }
    }
}

__global__ __launch_bounds__(256) void k_weak_copy(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                   const int32_t* __restrict__ idx, int32_t k,
                                                   uint16_t* __restrict__ ww)
{
    const int64_t total = N * k;
    for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < total; t += (int64_t)gridDim.x * 256) {
        const int64_t row = t / k, c = t % k;
        const int32_t j = idx[c];
        ww[t] = (j >= 0 && j < K) ? W[row * K + j] : (uint16_t)0;
    }
}

}  // namespace

bool grouped_size_supported(int64_t G, int64_t K)
{
    return G >= 32 && G <= 2048 && (G & (G - 1)) == 0 && K % G == 0;
}

hipError_t launch_pack_grouped(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k, int64_t G,
                               uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s)
{
    const int64_t waves = (N * (K / 32) + 63) / 64;
    const int64_t want = (waves + 3) / 4;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    const size_t lds = (size_t)(K / 32) * 4;
    // with k == 0 the weak-mask loop does not run; idx is never read
    switch (G) {
    case 32: hipLaunchKernelGGL((k_pack_grouped<1>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    case 64: hipLaunchKernelGGL((k_pack_grouped<2>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    case 128: hipLaunchKernelGGL((k_pack_grouped<4>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    case 256: hipLaunchKernelGGL((k_pack_grouped<8>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    case 512: hipLaunchKernelGGL((k_pack_grouped<16>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    case 1024: hipLaunchKernelGGL((k_pack_grouped<32>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    default: hipLaunchKernelGGL((k_pack_grouped<64>), dim3(blocks), dim3(256), lds, s, W, N, K, idx, k, q, scales, zeros); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || k == 0)
        return e;
    const int64_t wb = (N * k + 255) / 256;
    hipLaunchKernelGGL(k_weak_copy, dim3((unsigned)(wb < 4096 ? wb : 4096)), dim3(256), 0, s, W, N, K, idx, k, ww);
    return hipGetLastError();
}

}  // namespace owq
