// grouped.hip -- group-wise scales on top of OWQ (gfx950): pack and product.
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
// Product: a wavefront per output row, lane l taking code groups l, l + 64, ...;
// each group is decoded to exact (q - z) fp16 pairs (owq_decode.h) with its
// own zero point, its 16 v_dot2 run from 0, and the group's step scales that
// partial sum into the row's fp32 accumulator (one rounding). x comes straight
// from global memory (64 contiguous bytes per lane and token). The weak columns
// are added lane-strided, then a wave reduction and an fp16 store.
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

// Code groups per lane handled per batch of loads.
constexpr int kGroupsPerBatch = 2;

template <int M>
__global__ __launch_bounds__(256) void k_linear_grouped(const uint32_t* __restrict__ q,
                                                        const uint16_t* __restrict__ sc,
                                                        const uint8_t* __restrict__ zp,
                                                        const int32_t* __restrict__ idx,
                                                        const uint16_t* __restrict__ ww,
                                                        const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
                                                        int32_t N, int32_t K, int32_t k, int32_t G)
{
    const int lane = threadIdx.x & 63;
    const int row = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    if (row >= N)
        return;  // no block barrier below
    const int NC = K >> 5, CG = G >> 5, NG = K / G;
    const Magic mg = make_magic();
    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++)
        acc[m] = 0.0f;

    for (int c0 = 0; c0 < NC; c0 += 64 * kGroupsPerBatch) {
        u32x3 cw[kGroupsPerBatch];
        uint32_t sv[kGroupsPerBatch], zv[kGroupsPerBatch];
        uint4 xv[kGroupsPerBatch][M][4];
        bool on[kGroupsPerBatch];
        // every load of the batch first (clamped indices), then the arithmetic
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; u++) {
            const int cg = c0 + 64 * u + lane;
            on[u] = cg < NC;
            const int cgc = on[u] ? cg : NC - 1;
            const uint32_t* src = q + ((int64_t)row * NC + cgc) * 3;
            cw[u] = u32x3{src[0], src[1], src[2]};
            const int gi = cgc / CG;
            sv[u] = sc[(int64_t)row * NG + gi];
            zv[u] = zp[(int64_t)row * NG + gi];
#pragma unroll
            for (int m = 0; m < M; m++) {
                const uint4* xp = reinterpret_cast<const uint4*>(x + (int64_t)m * K + cgc * 32);
#pragma unroll
                for (int qd = 0; qd < 4; qd++)
                    xv[u][m][qd] = xp[qd];
            }
        }
#pragma unroll
        for (int u = 0; u < kGroupsPerBatch; u++) {
            if (!on[u])
                continue;
            const ZeroSub nz = make_zero_sub(zv[u]);
            uint32_t p[16];
            decode_group(cw[u].x, cw[u].y, cw[u].z, mg, nz, p);
            const float s = h2f((uint16_t)sv[u]);
#pragma unroll
            for (int m = 0; m < M; m++) {
                float part = 0.0f;
#pragma unroll
                for (int qd = 0; qd < 4; qd++) {
                    part = dot2(p[4 * qd + 0], xv[u][m][qd].x, part);
                    part = dot2(p[4 * qd + 1], xv[u][m][qd].y, part);
                    part = dot2(p[4 * qd + 2], xv[u][m][qd].z, part);
                    part = dot2(p[4 * qd + 3], xv[u][m][qd].w, part);
                }
                acc[m] = __builtin_fmaf(s, part, acc[m]);
            }
        }
    }
    // the weak columns: exact fp16 products, fp32 sums
    for (int c = lane; c < k; c += 64) {
        int j = idx[c];
        j = (j >= 0 && j < K) ? j : 0;
        const float w = h2f(ww[(int64_t)row * k + c]);
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[m] = __builtin_fmaf(w, h2f(x[(int64_t)m * K + j]), acc[m]);
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float t = wave_sum(acc[m]);
        if (lane == 0)
            y[(int64_t)m * N + row] = f2h(t);
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

hipError_t launch_linear_grouped(const LinearDesc& d, int64_t G, int64_t M, hipStream_t s)
{
    const unsigned blocks = (unsigned)((d.N + 3) / 4);
    // with no weak columns the weak arrays are never read; pass valid pointers anyway
    const int32_t* idx = d.k > 0 ? d.idx : reinterpret_cast<const int32_t*>(d.x);
    const uint16_t* ww = d.k > 0 ? d.ww : d.s;
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += kGroupedMaxM) {
        const int64_t mm = M - m0 < kGroupedMaxM ? M - m0 : kGroupedMaxM;
        const uint16_t* xm = d.x + m0 * d.K;
        uint16_t* ym = d.y + m0 * d.N;
#define OWQ_LG(MM)                                                                                         \
    hipLaunchKernelGGL((k_linear_grouped<MM>), dim3(blocks), dim3(256), 0, s, d.q, d.s, d.z, idx, ww, xm, ym, \
                       (int32_t)d.N, (int32_t)d.K, d.k, (int32_t)G)
        switch (mm) {
        case 1: OWQ_LG(1); break;
        case 2: OWQ_LG(2); break;
        case 3: OWQ_LG(3); break;
        default: OWQ_LG(4); break;
        }
#undef OWQ_LG
        e = hipGetLastError();
    }
    return e;
}

}  // namespace owq
