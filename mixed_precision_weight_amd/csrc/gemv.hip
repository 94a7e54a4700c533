// gemv.hip -- decode-time OWQ linear, small batch M (gfx950, vector ALUs).
//
//   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
//
// The 3-bit dense matrix is streamed once from HBM; the weak fp16 block is a
// small contiguous [N][k] array and only x is gathered at the weak indices, on
// the fly ([PL] "Real-device acceleration", paper "Acceleration on Real Device"
// p.6; [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models").
//
// Work split: a 256-thread block owns 4R consecutive rows (R per wavefront); the
// 64 lanes of a wave split each row's K/32 groups (lane l takes groups l, l+64,
// ...), so one wave load instruction reads 64 consecutive 12-byte groups (768
// contiguous bytes). The codes of a K chunk are all requested before x is
// staged, so their HBM latency overlaps the staging.
//
// Decode without per-code shifts: a 3-bit field that sits inside the mantissa of
// an fp16 half (bits p..p+2 with p <= 7) becomes an exact fp16 number once an
// exponent is OR-ed above it: exponent 2^(10-p) gives the value 2^(10-p) + q.
// With the sequential bit order (code c at bits 3c..3c+2 of the 96-bit group),
// six 32-bit windows of the group (w0>>2, bits 11..42, w1, w1>>9, bits 62..93,
// w2>>7) each hold codes at in-half positions 1/4/7 (low half) and 0/3/6 (high
// half), so one v_and_or_b32 yields a packed pair (off_lo + q_a, off_hi + q_b);
// codes 0 and 31 form the sixteenth pair. One v_pk_add_f16 of the row's
// -(off + z) pair then gives (q_a - z, q_b - z) EXACTLY (small integers), and one
// v_dot2_f32_f16 multiplies it with the matching x pair. Every product is exact,
// so the fp32 sum's error is bounded relative to sum_j |(q_j - z) x_j|, for
// every row, including rows whose codes all equal the zero point. Per group and
// row: 5 window ops, 17 and-or, 16 packed subtracts, 16 dot2 (about 1.7 VALU
// instructions per weight). x is staged once per block in LDS in this pair order.
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

struct GemvLayer {
    const uint32_t* q;
    const uint16_t* s;
    const uint8_t* z;
    const int32_t* idx;
    const uint16_t* ww;
    const uint16_t* x;
    uint16_t* y;
    int32_t N, K, k, block0;
};

struct GemvBatch {
    GemvLayer L[kGemvMaxLayers];
    int32_t count;
};

// Pair p of a group = (code lo[p], code hi[p]).
__device__ constexpr int kPairLo[16] = {1, 2, 3, 4, 5, 11, 12, 13, 14, 15, 21, 22, 23, 24, 25, 0};
__device__ constexpr int kPairHi[16] = {6, 7, 8, 9, 10, 16, 17, 18, 19, 20, 26, 27, 28, 29, 30, 31};

// Field masks and exponents: low-half positions 1/4/7 with exponents 2^9/2^6/2^3,
// high-half positions 0/3/6 with exponents 2^10/2^7/2^4 -> coefficient 1 on q.
constexpr uint32_t kMaskA = 0x0007000eu, kMagicA = 0x64006000u;  // (512 + q, 1024 + q)
constexpr uint32_t kMaskB = 0x00380070u, kMagicB = 0x58005400u;  // (64 + q, 128 + q)
constexpr uint32_t kMaskC = 0x01c00380u, kMagicC = 0x4c004800u;  // (8 + q, 16 + q)

struct U3 {
    uint32_t a, b, c;
};

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// v_and_or_b32 d = (a & mask) | magic. gfx9 VOP3 takes no literal operands and
// reads at most one SGPR, so the mask goes in an SGPR and the exponent pattern in
// a VGPR; plain C would be split into v_and_b32 + v_or_b32 with two literals.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic)
{
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(magic));
    return d;
}

struct Magic {  // exponent patterns held in VGPRs for the whole kernel
    uint32_t a, b, c, p;
};

__device__ __forceinline__ Magic make_magic()
{
    Magic m;
    // opaque to the optimiser so the constants stay in registers
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.a) : "i"(kMagicA));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.b) : "i"(kMagicB));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.c) : "i"(kMagicC));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.p) : "i"(0x64006400u));
    return m;
}

// -(off + z) for both halves of each pair type, as fp16 bit patterns:
// off + z = 2^E + z has mantissa field z * 2^(10 - E) under exponent E.
struct ZeroSub {
    uint32_t a, b, c, p;
};

__device__ __forceinline__ ZeroSub make_zero_sub(uint32_t z)
{
    ZeroSub n;
    n.a = ((0xe400u | z) << 16) | (0xe000u | (z << 1));          // -(1024 + z), -(512 + z)
    n.b = ((0xd800u | (z << 3)) << 16) | (0xd400u | (z << 4));   // -(128 + z),  -(64 + z)
    n.c = ((0xcc00u | (z << 6)) << 16) | (0xc800u | (z << 7));   // -(16 + z),   -(8 + z)
    n.p = ((0xe400u | z) << 16) | (0xe400u | z);                 // -(1024 + z) twice
    return n;
}

__device__ __forceinline__ uint32_t sub_h2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, as_h2(a) + as_h2(b));
}

// Sixteen exact (q_lo - z, q_hi - z) fp16 pairs of one 96-bit group, in
// kPairLo/kPairHi order.
__device__ __forceinline__ void decode_group(uint32_t w0, uint32_t w1, uint32_t w2, const Magic& mg,
                                             const ZeroSub& n, uint32_t p[16])
{
    const uint32_t a1 = w0 >> 2;
    const uint32_t b1 = __builtin_amdgcn_alignbit(w1, w0, 11);
    const uint32_t a2 = w1;
    const uint32_t b2 = w1 >> 9;
    const uint32_t a3 = __builtin_amdgcn_alignbit(w2, w1, 30);
    const uint32_t b3 = w2 >> 7;
    p[0] = sub_h2(and_or(a1, kMaskA, mg.a), n.a);
    p[1] = sub_h2(and_or(a1, kMaskB, mg.b), n.b);
    p[2] = sub_h2(and_or(a1, kMaskC, mg.c), n.c);
    p[3] = sub_h2(and_or(b1, kMaskA, mg.a), n.a);
    p[4] = sub_h2(and_or(b1, kMaskB, mg.b), n.b);
    p[5] = sub_h2(and_or(a2, kMaskA, mg.a), n.a);
    p[6] = sub_h2(and_or(a2, kMaskB, mg.b), n.b);
    p[7] = sub_h2(and_or(a2, kMaskC, mg.c), n.c);
    p[8] = sub_h2(and_or(b2, kMaskA, mg.a), n.a);
    p[9] = sub_h2(and_or(b2, kMaskB, mg.b), n.b);
    p[10] = sub_h2(and_or(a3, kMaskA, mg.a), n.a);
    p[11] = sub_h2(and_or(a3, kMaskB, mg.b), n.b);
    p[12] = sub_h2(and_or(a3, kMaskC, mg.c), n.c);
    p[13] = sub_h2(and_or(b3, kMaskA, mg.a), n.a);
    p[14] = sub_h2(and_or(b3, kMaskB, mg.b), n.b);
    // (1024 + q0, 1024 + q31): code 0 at bits 0..2 of w0, code 31 at bits 29..31 of w2
    p[15] = sub_h2(and_or(w2 >> 13, 0x00070000u, and_or(w0, 7u, mg.p)), n.p);
}

// Stage the 32 x values of one group as 16 pair words in decode order
// (4 x uint4 at stride GC).
template <int GC>
__device__ __forceinline__ void stage_group(const uint16_t* __restrict__ src, uint4* __restrict__ xs_mg)
{
    const uint4* p4 = reinterpret_cast<const uint4*>(src);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint4 t = p4[i];
        w[4 * i + 0] = t.x;
        w[4 * i + 1] = t.y;
        w[4 * i + 2] = t.z;
        w[4 * i + 3] = t.w;
    }
    uint32_t pr[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int lo = kPairLo[i], hi = kPairHi[i];
        uint32_t hl = (w[lo >> 1] >> (16 * (lo & 1))) & 0xffffu;
        uint32_t hh = (w[hi >> 1] >> (16 * (hi & 1))) & 0xffffu;
        pr[i] = hl | (hh << 16);
    }
#pragma unroll
    for (int qd = 0; qd < 4; qd++)
        xs_mg[qd * GC] = make_uint4(pr[4 * qd], pr[4 * qd + 1], pr[4 * qd + 2], pr[4 * qd + 3]);
}

template <int M, int R, int UPL>
__global__ __launch_bounds__(256) void k_gemv(GemvBatch b)
{
    constexpr int GC = 64 * UPL;  // groups per K chunk
    extern __shared__ uint4 xs[];  // [M][4][GC] pair quads

    int li = 0;
    for (int l = 1; l < b.count; l++)
        if ((int)blockIdx.x >= b.L[l].block0)
            li = l;
    const uint32_t* __restrict__ Q = b.L[li].q;
    const uint16_t* __restrict__ X = b.L[li].x;
    const int64_t N = b.L[li].N;
    const int64_t K = b.L[li].K;
    const int G = (int)(K / 32);
    const int64_t row0 = (int64_t)((int)blockIdx.x - b.L[li].block0) * (4 * R) + (threadIdx.x >> 6) * R;
    const int lane = threadIdx.x & 63;
    const Magic mg = make_magic();

    ZeroSub nz[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        nz[r] = make_zero_sub(row0 + r < N ? (uint32_t)b.L[li].z[row0 + r] : 0u);

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[r][m] = 0.0f;

    for (int gbase = 0; gbase < G; gbase += GC) {
        const int gc = min(GC, G - gbase);
        U3 cw[R][UPL];
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int u = 0; u < UPL; u++) {
                const int g = lane + 64 * u;
                const int64_t row = row0 + r;
                if (g < gc && row < N)
                    cw[r][u] = *reinterpret_cast<const U3*>(Q + (row * G + gbase + g) * 3);
                else
                    cw[r][u] = U3{0u, 0u, 0u};
            }
        __syncthreads();  // previous chunk's x no longer in use
        for (int i = threadIdx.x; i < M * gc; i += 256) {
            const int m = i / gc, g = i - m * gc;
            stage_group<GC>(X + (int64_t)m * K + (int64_t)(gbase + g) * 32, xs + (m * 4) * GC + g);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < UPL; u++) {
            const int g = lane + 64 * u;
            if (g < gc) {
                uint4 xq[M][4];
#pragma unroll
                for (int m = 0; m < M; m++)
#pragma unroll
                    for (int qd = 0; qd < 4; qd++)
                        xq[m][qd] = xs[(m * 4 + qd) * GC + g];
#pragma unroll
                for (int r = 0; r < R; r++) {
                    if (row0 + r < N) {
                        uint32_t p[16];
                        decode_group(cw[r][u].a, cw[r][u].b, cw[r][u].c, mg, nz[r], p);
#pragma unroll
                        for (int m = 0; m < M; m++) {
                            float a = acc[r][m];
#pragma unroll
                            for (int qd = 0; qd < 4; qd++) {
                                a = dot2(p[4 * qd + 0], xq[m][qd].x, a);
                                a = dot2(p[4 * qd + 1], xq[m][qd].y, a);
                                a = dot2(p[4 * qd + 2], xq[m][qd].z, a);
                                a = dot2(p[4 * qd + 3], xq[m][qd].w, a);
                            }
                            acc[r][m] = a;
                        }
                    }
                }
            }
        }
    }

    // epilogue: row scale, weak columns, wave reduction, fp16 store
    const uint16_t* __restrict__ SC = b.L[li].s;
    float part[R][M];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int64_t row = row0 + r;
        const float sf = row < N ? h2f(SC[row]) : 0.0f;
#pragma unroll
        for (int m = 0; m < M; m++)
            part[r][m] = sf * acc[r][m];
    }
    const int k = b.L[li].k;
    const int32_t* __restrict__ IDX = b.L[li].idx;
    const uint16_t* __restrict__ WW = b.L[li].ww;
    for (int c0 = 0; c0 < k; c0 += 64) {
        const int c = c0 + lane;
        const bool cv = c < k;
        int j = cv ? IDX[c] : 0;
        j = (j >= 0 && j < K) ? j : 0;
        float xv[M];
#pragma unroll
        for (int m = 0; m < M; m++)
            xv[m] = cv ? h2f(X[(int64_t)m * K + j]) : 0.0f;
#pragma unroll
        for (int r = 0; r < R; r++) {
            const int64_t row = row0 + r;
            if (cv && row < N) {
                const float w = h2f(WW[row * k + c]);
#pragma unroll
                for (int m = 0; m < M; m++)
                    part[r][m] += w * xv[m];
            }
        }
    }
    uint16_t* __restrict__ Y = b.L[li].y;
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float v = wave_sum(part[r][m]);
            if (lane == r * M + m && row0 + r < N)
                Y[(int64_t)m * N + row0 + r] = f2h(v);
        }
}

constexpr int kRows = 4;  // rows per wavefront

template <int M, int UPL>
hipError_t launch_t(const GemvBatch& b, int nblocks, hipStream_t s)
{
    const size_t lds = (size_t)M * 64 * UPL * 4 * sizeof(uint4);
    hipLaunchKernelGGL((k_gemv<M, kRows, UPL>), dim3(nblocks), dim3(256), lds, s, b);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const GemvBatch& b, int nblocks, int upl, hipStream_t s)
{
    // LDS per block = M * 64 * UPL * 64 bytes, kept under 33 KB:
    // UPL <= 8 for M = 1, <= 4 for M = 2, <= 2 for M = 3, 4. Larger K loops over chunks.
    if (upl <= 1)
        return launch_t<M, 1>(b, nblocks, s);
    if constexpr (M >= 3) {
        return launch_t<M, 2>(b, nblocks, s);
    } else if constexpr (M == 2) {
        if (upl <= 2)
            return launch_t<M, 2>(b, nblocks, s);
        return launch_t<M, 4>(b, nblocks, s);
    } else {
        if (upl <= 2)
            return launch_t<M, 2>(b, nblocks, s);
        if (upl <= 4)
            return launch_t<M, 4>(b, nblocks, s);
        if (upl <= 6)
            return launch_t<M, 6>(b, nblocks, s);
        return launch_t<M, 8>(b, nblocks, s);
    }
}

}  // namespace

hipError_t launch_gemv(const LinearDesc* d, int count, int M, hipStream_t s)
{
    GemvBatch b{};
    b.count = count;
    int nblocks = 0;
    int64_t gmax = 0;
    for (int l = 0; l < count; l++) {
        GemvLayer& L = b.L[l];
        L.q = d[l].q;
        L.s = d[l].s;
        L.z = d[l].z;
        L.idx = d[l].idx;
        L.ww = d[l].ww;
        L.x = d[l].x;
        L.y = d[l].y;
        L.N = (int32_t)d[l].N;
        L.K = (int32_t)d[l].K;
        L.k = d[l].k;
        L.block0 = nblocks;
        nblocks += (int)((d[l].N + 4 * kRows - 1) / (4 * kRows));
        gmax = d[l].K / 32 > gmax ? d[l].K / 32 : gmax;
    }
    const int upl = (int)((gmax + 63) / 64);
    switch (M) {
    case 1: return launch_m<1>(b, nblocks, upl, s);
    case 2: return launch_m<2>(b, nblocks, upl, s);
    case 3: return launch_m<3>(b, nblocks, upl, s);
    default: return launch_m<4>(b, nblocks, upl, s);
    }
}

}  // namespace owq
