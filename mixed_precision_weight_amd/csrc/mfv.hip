// mfv.hip -- decode-time OWQ linear on the matrix cores, 1 <= M <= 16 (gfx950).
//
//   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
//
// The 3-bit dense matrix is streamed once from HBM and decoded in registers;
// the weak fp16 block is contiguous and only x is gathered at the weak indices
// ([PL] "Real-device acceleration", paper "Acceleration on Real Device" p.6;
// [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models").
//
// Why the matrix cores for several tokens: the register decode of a 32-code
// group costs 39 vector instructions per lane, and a vector multiply-accumulate
// with x would add 16 v_dot2 per token on top. Here v_mfma_f32_16x16x32_f16 does
// the products for up to 16 tokens at once, so the vector ALUs only decode and
// the cost per weight does not grow with the token count.
//
// Lane layout: the MFMA pairs the 8 operand elements of lane l with the k values
// 8 (l / 16) + e, for A row (token) l % 16 and B column (output row) l % 16.
// A wavefront owns 16 consecutive output rows: lane l decodes, for row l % 16,
// the groups 4 u + l / 16 (u < U) of each K chunk of 4 U groups, so each load
// instruction of the wave reads 48 contiguous bytes from each of its 16 rows;
// the 16 decode pairs of a group feed four MFMA steps (pairs 4t .. 4t + 3 in
// step t). Decode pair p is columns (2p, 2p + 1) (the slot layout of the codes),
// so x is staged as it is stored: the block's x chunk sits in LDS as
// [token][group][32 values] and an A operand is one 128-bit LDS read per lane.
// The K reduction happens inside the accumulators: no cross-lane reduction.
//
// Pipeline: LDS double buffer for x, the next chunk's codes and x in registers
// while the current chunk computes, one barrier per chunk. A block is 4 waves
// (64 rows) of one layer; one launch covers a batch of layers of any shapes.
// Epilogue: row step, the weak columns as extra 32-deep MFMA steps (fp16 weak
// weights against x gathered at weak_idx), fp16 stores.
#include <cstdlib>
#include <cstring>

#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct MfvLayer {
    const uint32_t* q;
    const uint16_t* s;
    const uint8_t* z;
    const int32_t* idx;
    const uint16_t* ww;
    const uint16_t* x;
    uint16_t* y;
    int32_t N, K, k;
    int32_t block0;  // first block of this layer
};

struct MfvBatch {
    MfvLayer L[kGemvMaxLayers];
    int32_t count;
};

constexpr int kRowsPerBlock = 64;

__device__ __forceinline__ half8_t h8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(half8_t, make_uint4(a, b, c, d));
}

// U groups per lane per chunk; MC = largest token count of the instance.
template <int U, int MC>
struct MfvShape {
    static constexpr int GC = 4 * U;                     // groups per chunk
    static constexpr int RS = GC * 64 + 16;              // LDS bytes per staged token (padded)
    static constexpr int XI = (MC * GC + 255) / 256;     // staged group rows per thread
    static constexpr int LDS = 2 * MC * RS;              // double buffer
};

template <int U, int MC>
__global__ __launch_bounds__(256) void k_mfv(MfvBatch b, int M)
{
    using S = MfvShape<U, MC>;
    constexpr int GC = S::GC, RS = S::RS, XI = S::XI;
    extern __shared__ uint4 smem[];
    char* const lds = reinterpret_cast<char*>(smem);

    int li = 0;
    for (int l = 1; l < b.count; l++)
        if ((int)blockIdx.x >= b.L[l].block0)
            li = l;
    const MfvLayer& L = b.L[li];
    const int N = L.N, K = L.K, k = L.k;
    const int G = K >> 5;
    const int nch = (G + GC - 1) / GC;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, qd = lane >> 4;
    const int brow = ((int)blockIdx.x - L.block0) * kRowsPerBlock;
    const int nb = min(N - brow, kRowsPerBlock);  // valid rows of the block
    const int rloc = min(wave * 16 + l16, nb - 1);  // this lane's row in the block (clamped)

    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(L.q) + (int64_t)brow * G * 3, (short)0, nb * G * 12, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(L.x), (short)0, M * K * 2, 0x00020000);
    const int qrow = rloc * G * 12;

    // staging items i = tid + 256 t: token i / GC, group i % GC of the chunk
    i32x4 xg[XI][4];
    u32x3 cw[U];
    auto issue = [&](int c) {
#pragma unroll
        for (int t = 0; t < XI; t++) {
            const int i = tid + 256 * t;
            const int m = min(i / GC, M - 1);
            const int g = min(c * GC + i % GC, G - 1);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                xg[t][q4] = __builtin_amdgcn_raw_buffer_load_b128(xr, (m * K + g * 32) * 2 + 16 * q4, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int g = min(c * GC + 4 * u + qd, G - 1);
            cw[u] = __builtin_amdgcn_raw_buffer_load_b96(qr, qrow + g * 12, 0, 0);
        }
    };
    auto stage = [&](int c) {
        char* const buf = lds + (c & 1) * MC * RS;
#pragma unroll
        for (int t = 0; t < XI; t++) {
            const int i = tid + 256 * t;
            if (i < M * GC) {
                const bool live = c * GC + i % GC < G;
                uint32_t pr[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        pr[4 * q4 + e] = live ? (uint32_t)xg[t][q4][e] : 0u;
                uint4* dst = reinterpret_cast<uint4*>(buf + (i / GC) * RS + (i % GC) * 64);
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
                    dst[q4] = make_uint4(pr[4 * q4], pr[4 * q4 + 1], pr[4 * q4 + 2], pr[4 * q4 + 3]);
            }
        }
    };

    const float sc = h2f(L.s[brow + rloc]);
    const ZeroSub zs = make_zero_sub((uint32_t)L.z[brow + rloc]);
    const Magic mg = make_magic();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};

    issue(0);
    stage(0);
    __syncthreads();
    // this lane's A operand: token min(l16, M - 1), groups 4 u + qd of the chunk
    const int arow = min(l16, M - 1) * RS + qd * 64;
    for (int c = 0; c < nch; c++) {
        u32x3 cur[U];
#pragma unroll
        for (int u = 0; u < U; u++)
            cur[u] = cw[u];
        issue(min(c + 1, nch - 1));
        const char* const buf = lds + (c & 1) * MC * RS + arow;
#pragma unroll
        for (int u = 0; u < U; u++) {
            uint32_t p[16];
            decode_group(cur[u].x, cur[u].y, cur[u].z, mg, zs, p);
#pragma unroll
            for (int st = 0; st < 4; st++) {
                const half8_t av =
                    __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(buf + 4 * u * 64 + st * 16));
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    av, h8_of(p[4 * st], p[4 * st + 1], p[4 * st + 2], p[4 * st + 3]), acc, 0, 0, 0);
            }
        }
        if (c + 1 < nch)
            stage(c + 1);
        __syncthreads();
    }

    // row step, then the weak columns: B = w_weak[row][cs + 8 qd + e], A = x[token][idx[...]]
#pragma unroll
    for (int r = 0; r < 4; r++)
        acc[r] *= sc;
    if (k > 0) {
        const uint16_t* wr = L.ww + (int64_t)(brow + rloc) * k;
        const uint16_t* xm = L.x + (int64_t)min(l16, M - 1) * K;
        for (int cs = 0; cs < k; cs += 32) {
            uint32_t bw[4], aw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) {
                uint32_t wv[2], xv[2];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int c = cs + 8 * qd + 2 * e2 + h;
                    const bool on = c < k;
                    int j = L.idx[min(c, k - 1)];
                    j = (j >= 0 && j < K) ? j : 0;
                    wv[h] = on ? (uint32_t)wr[min(c, k - 1)] : 0u;
                    xv[h] = on ? (uint32_t)xm[j] : 0u;
                }
                bw[e2] = wv[0] | (wv[1] << 16);
                aw[e2] = xv[0] | (xv[1] << 16);
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(h8_of(aw[0], aw[1], aw[2], aw[3]),
                                                        h8_of(bw[0], bw[1], bw[2], bw[3]), acc, 0, 0, 0);
        }
    }

    // D element r of lane l: token 4 (l / 16) + r, row l % 16
    const int row = wave * 16 + l16;
    if (row < nb) {
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int m = 4 * qd + r;
            if (m < M)
                L.y[(int64_t)m * N + brow + row] = f2h(acc[r]);
        }
    }
}

template <int U, int MC>
hipError_t launch_shape(const MfvBatch& b, int nblocks, int M, hipStream_t s)
{
    using S = MfvShape<U, MC>;
    hipLaunchKernelGGL((k_mfv<U, MC>), dim3(nblocks), dim3(256), S::LDS, s, b, M);
    return hipGetLastError();
}

}  // namespace

bool decode_on_matrix_cores(int64_t M)
{
    const char* e = std::getenv("OWQ_DECODE");
    if (e && std::strcmp(e, "vector") == 0)
        return M > kGemvMaxM;
    if (e && std::strcmp(e, "matrix") == 0)
        return true;
    return M > kGemvMaxM;
}

bool mfv_fits(int64_t M, int64_t K)
{
    return M >= 1 && M <= kMfvMaxM && M * K * 2 <= INT32_MAX;
}

hipError_t launch_mfv(const LinearDesc* d, int count, int M, hipStream_t s)
{
    // layers with the longest rows first: their blocks run longest
    int order[kGemvMaxLayers];
    for (int l = 0; l < count; l++)
        order[l] = l;
    for (int a = 1; a < count; a++)
        for (int c = a; c > 0 && d[order[c]].K > d[order[c - 1]].K; c--) {
            const int t = order[c];
            order[c] = order[c - 1];
            order[c - 1] = t;
        }
    MfvBatch b{};
    int nblocks = 0;
    for (int o = 0; o < count; o++) {
        const LinearDesc& dl = d[order[o]];
        MfvLayer& L = b.L[b.count++];
        L.q = dl.q;
        L.s = dl.s;
        L.z = dl.z;
        L.idx = dl.idx;
        L.ww = dl.ww;
        L.x = dl.x;
        L.y = dl.y;
        L.N = (int32_t)dl.N;
        L.K = (int32_t)dl.K;
        L.k = dl.k;
        L.block0 = nblocks;
        nblocks += (int)((dl.N + kRowsPerBlock - 1) / kRowsPerBlock);
    }
    if (M <= 4)
        return launch_shape<4, 4>(b, nblocks, M, s);
    return launch_shape<4, 16>(b, nblocks, M, s);
}

}  // namespace owq
