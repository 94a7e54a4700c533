// search.hip -- truncation-aware choice of each row's step size and zero point
// (gfx950).
//
// Before the dense columns are quantised, the step size and zero point of each
// output row come from a 2D grid search over both, with round-to-nearest codes
// clamped to the 3-bit range, so that a range narrower than min-max can win by
// truncating a few large weights ([PL] "Low-precision quantization", paper
// "Quantization Configuration Search", pp.4-5; [PL] = paperlayer.ai page "OWQ:
// Outlier-Aware Weight Quantization for Efficient Fine-Tuning and Inference of
// Large Language Models"). The grid and the objective:
//   steps   s_a = fp16(s_mm * (1 - a/40)), a = 0..31, s_mm = (hi - lo) / 7 the
//           fp32 min-max step over the row's dense columns (0 inside [lo, hi]);
//           a step that rounds to fp16 zero is skipped;
//   zeros   z = 0..7;
//   error   E(a, z) = sum over dense columns j, ascending, of
//           omega_j (w_j - s_a (clamp(rint(w_j / s_a) + z, 0, 7) - z))^2,
//           omega_j = lambda_j (the Hessian diagonal) or 1, in fp64;
//   choice  the smallest E, ties to the smaller a, then the smaller z;
//   a row with hi == lo, or whose min-max step rounds to fp16 zero, keeps step 1
//   and zero point 0.
//
// Kernel shape (ALU-bound): one 256-thread block per row (grid-stride); thread t
// evaluates grid point (a, z) = (t / 8, t % 8) over the whole row, so every
// error is ONE sequential fp64 sum in column order, the same sum as the
// definition's, bit for bit, and the argmin is decided on identical numbers.
// The row (weak entries zeroed: 0 lies in every fitted range and its term is an
// exact +0) and lambda are staged in LDS in chunks of kChunk columns; all 256
// threads read the same LDS words (broadcast). Per element a thread does one
// fp32 multiply and rint, a clamp, and four fp64 operations (d = w - s q by one
// exact FMA, d * d, lambda times it, the running sum). The rounding uses the
// reciprocal of the step: rint(w * rcp(s)) equals rint(w / s) except possibly at
// an exact half-integer, where both neighbours leave |d| = s / 2 (and the clamp
// maps an out-of-range neighbour onto the in-range one), so every term is the
// definition's. The winning (s, z) is written to scales / zeros, from which the
// pack kernels then emit the codes (with exact ties-to-even rounding).
//
// Built with -ffp-contract=off: every fp32 and fp64 step is one IEEE operation.
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kChunk = 2048;     // columns staged per pass
constexpr int kStepsSearched = 32;
constexpr int kCandidates = kStepsSearched * 8;  // one per thread

// fp16 step of grid point a: the fp32 product s_mm (1 - a/40), rounded to fp16.
// The product is pinned to a register first: otherwise the compiler folds the
// multiply and the conversion into one mixed-precision FMA that rounds the exact
// product straight to fp16, which differs from rounding the fp32 product.
__device__ __forceinline__ uint16_t grid_step(float s_mm, int a)
{
    const float f = 1.0f - (float)a / 40.0f;
    float p = s_mm * f;
    asm volatile("" : "+v"(p));
    return f2h(p);
}

template <bool kWeighted>
__global__ __launch_bounds__(256) void k_search(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                const int32_t* __restrict__ idx, int32_t k,
                                                const double* __restrict__ lam,
                                                uint16_t* __restrict__ scales, uint8_t* __restrict__ zeros)
{
    extern __shared__ uint32_t wmask[];  // [G] weak-column bit mask per 32-column group
    __shared__ uint4 wrow[kChunk / 8];   // the chunk's weights, weak entries zeroed
    __shared__ double lrow[kWeighted ? kChunk : 1];
    __shared__ float red[2][4];
    __shared__ double bestE[4];
    __shared__ int bestT[4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t G = K / 32;

    for (int64_t g = tid; g < G; g += 256)
        wmask[g] = 0;
    __syncthreads();
    for (int64_t c = tid; c < k; c += 256) {
        const int32_t j = idx[c];
        if (j >= 0 && j < K)  // indices outside [0, K) break the caller contract; never touch memory with them
            atomicOr(&wmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    // the 16-byte piece p of a row (8 columns) with its weak entries zeroed
    auto piece = [&](const uint16_t* wr, int64_t p) {
        uint4 v = *reinterpret_cast<const uint4*>(wr + p * 8);
        const uint32_t m = (wmask[p >> 2] >> ((p & 3) * 8)) & 0xffu;
        uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
            if (m & (1u << (2 * i)))
                h[i] &= 0xffff0000u;
            if (m & (2u << (2 * i)))
                h[i] &= 0x0000ffffu;
        }
        return make_uint4(h[0], h[1], h[2], h[3]);
    };

    const int a = tid >> 3, zc = tid & 7;
    for (int64_t row = blockIdx.x; row < N; row += gridDim.x) {
        const uint16_t* wr = W + row * K;
        // min-max range of the dense columns, 0 included
        float lo = 0.0f, hi = 0.0f;
        for (int64_t p = tid; p < K / 8; p += 256) {
            const uint4 v = piece(wr, p);
            const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float f = h2f((uint16_t)(h[i >> 1] >> (16 * (i & 1))));
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
        const float s_mm = (hi - lo) / 7.0f;
        const bool degenerate = hi == lo || (f2h(s_mm) & 0x7fff) == 0;  // block-uniform
        if (degenerate) {
            if (tid == 0) {
                scales[row] = 0x3c00;
                zeros[row] = 0;
            }
            __syncthreads();  // red[] is reused by the next row
            continue;
        }
        const uint16_t sa = grid_step(s_mm, a);
        const bool valid = (sa & 0x7fff) != 0;
        const float sf = valid ? h2f(sa) : 1.0f;
        const float rs = __builtin_amdgcn_rcpf(sf);
        const double sd = (double)sf;
        const float qlo = -(float)zc, qhi = 7.0f - (float)zc;

        double E = 0.0;
        for (int64_t c0 = 0; c0 < K; c0 += kChunk) {
            const int n = (int)min((int64_t)kChunk, K - c0);  // multiple of 32
            __syncthreads();  // the previous chunk is no longer read
            for (int p = tid; p < n / 8; p += 256)
                wrow[p] = piece(wr, c0 / 8 + p);
            if (kWeighted)
                for (int j = tid; j < n; j += 256)
                    lrow[j] = lam[c0 + j];
            __syncthreads();
            for (int p = 0; p < n / 8; p++) {
                const uint4 v = wrow[p];  // the same word in every lane
                const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float w = h2f((uint16_t)(h[i >> 1] >> (16 * (i & 1))));
                    const float q = __builtin_amdgcn_fmed3f(rintf(w * rs), qlo, qhi);
                    const double d = __builtin_fma(-sd, (double)q, (double)w);  // exact
                    double t = d * d;
                    if (kWeighted)
                        t = lrow[8 * p + i] * t;
                    E += t;
                }
            }
        }
        if (!valid)
            E = __builtin_inf();

        // argmin of (E, thread): the thread order is the grid's (a, then z)
        int bt = tid;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const double e2 = shfl_xor_f64(E, o);
            const int t2 = __shfl_xor(bt, o, 64);
            if (e2 < E || (e2 == E && t2 < bt)) {
                E = e2;
                bt = t2;
            }
        }
        if (lane == 0) {
            bestE[wave] = E;
            bestT[wave] = bt;
        }
        __syncthreads();
        if (tid == 0) {
            double be = bestE[0];
            int b = bestT[0];
            for (int w = 1; w < 4; w++)
                if (bestE[w] < be) {  // later waves hold later grid points: strict
                    be = bestE[w];
                    b = bestT[w];
                }
            scales[row] = grid_step(s_mm, b >> 3);
            zeros[row] = (uint8_t)(b & 7);
        }
        __syncthreads();  // red[], bestE[] are reused by the next row
    }
}

}  // namespace

hipError_t launch_search(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                         const double* lambda, uint16_t* scales, uint8_t* zeros, hipStream_t s)
{
    static_assert(kCandidates == 256, "one grid point per thread");
    const int64_t G = K / 32;
    const unsigned grid = (unsigned)(N < 8192 ? N : 8192);
    const size_t lds = (size_t)G * sizeof(uint32_t);
    if (lambda)
        hipLaunchKernelGGL(k_search<true>, dim3(grid), dim3(256), lds, s, W, N, K, idx, k, lambda, scales,
                           zeros);
    else
        hipLaunchKernelGGL(k_search<false>, dim3(grid), dim3(256), lds, s, W, N, K, idx, k, lambda, scales,
                           zeros);
    return hipGetLastError();
}

}  // namespace owq
