// backward.hip -- backward of the OWQ linear for weak-column tuning (gfx950).
//
// Weak Column Tuning trains only the fp16 weak columns and keeps the 3-bit dense
// matrix frozen ([PL] "Weak Column Tuning", paper "PEFT with Weak Column
// Tuning" p.5; the trainable block is the N x k weak block, "Learnable
// Parameters", appendix section 3 p.13; [PL] = paperlayer.ai page "OWQ:
// Outlier-Aware Weight Quantization for Efficient Fine-Tuning and Inference of
// Large Language Models"). For y = x W^T, with W the dequantised dense matrix
// (0 at the weak columns) plus the weak columns, and an upstream gradient dy:
//   dx[m][j]      = sum_i dy[m][i] W[i][j]          (fp32 sums, fp16 result)
//   dw_weak[i][c] = sum_m dy[m][i] x[m][idx_c]      (fp32 sums, fp32 result)
//
// dx is the transposed 3-bit product: the reduction runs over the rows of the
// packed matrix, whose codes lie along K. k_bwd_dx_part streams the codes once
// per token chunk: a block is 4 waves over one tile of 64 groups (2048 columns)
// and one slice of rows; lane l decodes group l of the tile (the R7 slot layout
// gives natural column pairs) and adds s_i dy[m][i] (q_ij - z_i) into 32
// fp32 accumulators per token, one mixed-precision FMA per weight and token (the
// fp16 (q - z) is exact). Each wave writes its partial sums; k_bwd_weak_part sums
// dy w_weak over the same row slices for the weak columns (the dense codes there
// dequantise to 0), and k_bwd_dx_finalize adds the slices in a fixed order and
// rounds to fp16: results are bitwise deterministic. Token chunks of up to 4.
//
// dw_weak (k_bwd_dw): a thread per row and 32 weak columns, x at the weak
// columns staged in LDS 64 tokens at a time, fp32 FMAs in token order.
#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kBwdMaxMT = 4;      // tokens per dx pass
constexpr int kTileGroups = 64;   // groups per column tile (one per lane)
constexpr int kWeakTile = 32;     // weak columns per block in the weak kernels

// partial sums of one token chunk over one row slice, per wave:
// P[(slice * 4 + wave)][m][K] (fp32)
template <int MT>
__global__ __launch_bounds__(256) void k_bwd_dx_part(const uint32_t* __restrict__ q,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros, int N, int K,
                                                     const uint16_t* __restrict__ dy, int rows_per_slice,
                                                     float* __restrict__ P)
{
    const int G = K >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = blockIdx.x * kTileGroups + lane;
    const int gc = min(g, G - 1);  // lanes past the row's groups load a valid group and store nothing
    const int s = blockIdx.y;
    const int r0 = s * rows_per_slice, r1 = min(N, r0 + rows_per_slice);
    const Magic mg = make_magic();

    float acc[MT][32];
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
        for (int c = 0; c < 32; c++)
            acc[m][c] = 0.0f;

    for (int r = r0 + wave; r < r1; r += 4) {
        const uint32_t* src = q + ((int64_t)r * G + gc) * 3;
        const uint32_t w0 = src[0], w1 = src[1], w2 = src[2];
        const float sc = h2f(scales[r]);
        const uint32_t z = zeros[r];
        float coef[MT];
#pragma unroll
        for (int m = 0; m < MT; m++)
            coef[m] = sc * h2f(dy[(int64_t)m * N + r]);
        uint32_t p[16];
        decode_group(w0, w1, w2, mg, make_zero_sub(z), p);
#pragma unroll
        for (int pp = 0; pp < 16; pp++) {
            const half2_t h = as_h2(p[pp]);
            const float lo = (float)h.x, hi = (float)h.y;  // exact small integers
#pragma unroll
            for (int m = 0; m < MT; m++) {
                acc[m][2 * pp] = __builtin_fmaf(coef[m], lo, acc[m][2 * pp]);
                acc[m][2 * pp + 1] = __builtin_fmaf(coef[m], hi, acc[m][2 * pp + 1]);
            }
        }
    }
    if (g < G) {
        float* dst = P + ((int64_t)(s * 4 + wave) * MT) * K + (int64_t)g * 32;
#pragma unroll
        for (int m = 0; m < MT; m++)
#pragma unroll
            for (int c = 0; c < 32; c += 4)
                *reinterpret_cast<float4*>(dst + (int64_t)m * K + c) =
                    make_float4(acc[m][c], acc[m][c + 1], acc[m][c + 2], acc[m][c + 3]);
    }
}

// the weak columns' share of dx over one row slice: PW[slice][m][c] =
// sum_{i in slice} dy[m][i] w_weak[i][c]; 8 row phases x 32 columns per block,
// the phases added in a fixed order
template <int MT>
__global__ __launch_bounds__(256) void k_bwd_weak_part(const uint16_t* __restrict__ ww, int N, int k,
                                                       const uint16_t* __restrict__ dy, int rows_per_slice,
                                                       float* __restrict__ PW)
{
    __shared__ float red[8][MT][kWeakTile];
    const int cc = threadIdx.x & 31, ph = threadIdx.x >> 5;
    const int c = blockIdx.x * kWeakTile + cc;
    const int s = blockIdx.y;
    const int r0 = s * rows_per_slice, r1 = min(N, r0 + rows_per_slice);
    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; m++)
        acc[m] = 0.0f;
    if (c < k) {
        for (int r = r0 + ph; r < r1; r += 8) {
            const float w = h2f(ww[(int64_t)r * k + c]);
#pragma unroll
            for (int m = 0; m < MT; m++)
                acc[m] = __builtin_fmaf(h2f(dy[(int64_t)m * N + r]), w, acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < MT; m++)
        red[ph][m][cc] = acc[m];
    __syncthreads();
    if (ph == 0 && c < k) {
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float t = red[0][m][cc];
            for (int q2 = 1; q2 < 8; q2++)
                t += red[q2][m][cc];
            PW[((int64_t)s * MT + m) * k + c] = t;
        }
    }
}

// dx[m][j] = fp16(sum over the dense partials in order + the weak partials at
// weak columns)
__global__ __launch_bounds__(256) void k_bwd_dx_finalize(const float* __restrict__ P, int nparts,
                                                         const float* __restrict__ PW, int nweak_parts, int MT,
                                                         int K, const int32_t* __restrict__ idx, int k,
                                                         uint16_t* __restrict__ dx)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // m * K + j within the chunk
    if (e >= (int64_t)MT * K)
        return;
    const int m = (int)(e / K), j = (int)(e % K);
    float t = 0.0f;
    for (int s = 0; s < nparts; s++)
        t += P[((int64_t)s * MT + m) * K + j];
    // the weak column j, if any: binary search in the ascending indices
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] < j)
            lo = mid + 1;
        else
            hi = mid;
    }
    if (lo < k && idx[lo] == j) {
        float w = 0.0f;
        for (int s = 0; s < nweak_parts; s++)
            w += PW[((int64_t)s * MT + m) * k + lo];
        t += w;
    }
    dx[(int64_t)m * K + j] = f2h(t);
}

// dw[i][c] = sum_m dy[m][i] x[m][idx_c]: thread per row, 32 weak columns per block
__global__ __launch_bounds__(256) void k_bwd_dw(const uint16_t* __restrict__ x, int M, int K,
                                                const int32_t* __restrict__ idx, int k,
                                                const uint16_t* __restrict__ dy, int N, float* __restrict__ dw)
{
    constexpr int MC = 64;
    __shared__ float xw[MC][kWeakTile];
    const int i = blockIdx.x * 256 + threadIdx.x;
    const int c0 = blockIdx.y * kWeakTile;
    const int ic = min(i, N - 1);
    float acc[kWeakTile];
#pragma unroll
    for (int c = 0; c < kWeakTile; c++)
        acc[c] = 0.0f;
    for (int m0 = 0; m0 < M; m0 += MC) {
        __syncthreads();  // the previous tokens' x is no longer read
        for (int e = threadIdx.x; e < MC * kWeakTile; e += 256) {
            const int mm = e / kWeakTile, cc = e % kWeakTile;
            float v = 0.0f;
            if (m0 + mm < M && c0 + cc < k) {
                int j = idx[c0 + cc];
                j = (j >= 0 && j < K) ? j : 0;
                v = h2f(x[(int64_t)(m0 + mm) * K + j]);
            }
            xw[mm][cc] = v;
        }
        __syncthreads();
        const int mn = min(MC, M - m0);
        for (int mm = 0; mm < mn; mm++) {
            const float d = h2f(dy[(int64_t)(m0 + mm) * N + ic]);
#pragma unroll
            for (int c = 0; c < kWeakTile; c++)
                acc[c] = __builtin_fmaf(d, xw[mm][c], acc[c]);
        }
    }
    if (i < N)
        for (int c = 0; c < kWeakTile && c0 + c < k; c++)
            dw[(int64_t)i * k + c0 + c] = acc[c];
}

template <int MT>
hipError_t dx_chunk(const LinearDesc& d, const uint16_t* dy, uint16_t* dx, const BwdPlan& p, char* ws,
                    hipStream_t s)
{
    float* P = reinterpret_cast<float*>(ws + p.off_p);
    float* PW = reinterpret_cast<float*>(ws + p.off_pw);
    const int G = (int)(d.K / 32);
    const int tiles = (G + kTileGroups - 1) / kTileGroups;
    hipLaunchKernelGGL((k_bwd_dx_part<MT>), dim3(tiles, (unsigned)p.slices), dim3(256), 0, s, d.q, d.s, d.z,
                       (int)d.N, (int)d.K, dy, (int)p.rows_per_slice, P);
    if (d.k > 0)
        hipLaunchKernelGGL((k_bwd_weak_part<MT>), dim3((d.k + kWeakTile - 1) / kWeakTile, (unsigned)p.slices),
                           dim3(256), 0, s, d.ww, (int)d.N, d.k, dy, (int)p.rows_per_slice, PW);
    const int64_t n = (int64_t)MT * d.K;
    hipLaunchKernelGGL(k_bwd_dx_finalize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, P,
                       (int)(4 * p.slices), PW, d.k > 0 ? (int)p.slices : 0, MT, (int)d.K, d.idx, d.k, dx);
    return hipGetLastError();
}

}  // namespace

BwdPlan bwd_plan(int64_t N, int64_t K, int32_t k)
{
    BwdPlan p;
    // row slices of at least 64 rows (16 per wave), at most 64 slices, and the
    // dense partial sums (4 per slice, 4 tokens, K columns, fp32) within 32 MiB
    int64_t sl = (N + 63) / 64;
    const int64_t cap = ((int64_t)32 << 20) / (4 * kBwdMaxMT * K * (int64_t)sizeof(float));
    if (sl > 64)
        sl = 64;
    if (sl > cap)
        sl = cap;
    p.slices = sl < 1 ? 1 : sl;
    p.rows_per_slice = (N + p.slices - 1) / p.slices;
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    p.off_p = 0;
    p.off_pw = al((size_t)4 * p.slices * kBwdMaxMT * K * sizeof(float));
    p.total = p.off_pw + al((size_t)p.slices * kBwdMaxMT * (k > 0 ? k : 1) * sizeof(float));
    return p;
}

hipError_t launch_linear_backward(const LinearDesc& d, const uint16_t* dy, int64_t M, uint16_t* dx, float* dw,
                                  void* ws, const BwdPlan& p, hipStream_t s)
{
    hipError_t e = hipSuccess;
    if (dx) {
        char* w = static_cast<char*>(ws);
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += kBwdMaxMT) {
            const int mt = (int)(M - m0 < kBwdMaxMT ? M - m0 : kBwdMaxMT);
            const uint16_t* dyc = dy + m0 * d.N;
            uint16_t* dxc = dx + m0 * d.K;
            switch (mt) {
            case 1: e = dx_chunk<1>(d, dyc, dxc, p, w, s); break;
            case 2: e = dx_chunk<2>(d, dyc, dxc, p, w, s); break;
            case 3: e = dx_chunk<3>(d, dyc, dxc, p, w, s); break;
            default: e = dx_chunk<4>(d, dyc, dxc, p, w, s); break;
            }
        }
    }
    if (e == hipSuccess && dw && d.k > 0) {
        hipLaunchKernelGGL(k_bwd_dw, dim3((unsigned)((d.N + 255) / 256), (unsigned)((d.k + kWeakTile - 1) / kWeakTile)),
                           dim3(256), 0, s, d.x, (int)M, (int)d.K, d.idx, d.k, dy, (int)d.N, dw);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace owq
