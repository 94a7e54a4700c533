// gemm.hip -- prefill-time OWQ linear, larger batch M (gfx950 matrix cores).
//
//   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
//
// The 3-bit matrix is dequantised on the fly and multiplied on the matrix cores
// in fp16 with fp32 accumulation; the weak columns are a small dense fp16 block
// applied to x gathered at the weak indices ([PL] "Real-device acceleration",
// paper "Acceleration on Real Device" p.6; [PL] = paperlayer.ai page "OWQ:
// Outlier-Aware Weight Quantization for Efficient Fine-Tuning and Inference of
// Large Language Models").
//
// Tiling: a block owns a BM x BN tile of y (tokens x output rows) and its waves
// form a WM x WN grid, each wave owning 32 FM tokens x 32 FN rows, i.e. FM x FN
// accumulators of v_mfma_f32_32x32x16_f16 (A = x, B = the weights transposed).
// K is walked in chunks of 64 columns (two 32-code groups). From 128 tokens on
// the tile is 128 tokens x 256 rows, 4 waves of 64 x 128 and two blocks per CU
// (k_gemm_dma); below, 32 tokens x 256 rows, 4 waves of 32 x 64 (k_gemm).
//
// The weights never pass through LDS. The MFMA pairs the eight A and B operand
// elements of lane l with the same eight k values of half h = l / 32, and the
// order of a contraction is free, so lane l of a wave decodes group (chunk, h) of
// row l % 32 of each of its row blocks (owq_decode.h) straight into B operand
// registers: the 32 exact (q - z) values of the group feed the chunk's four
// 16-deep MFMA steps, four decode pairs (8 consecutive columns) per step.
// x goes through LDS as stored (decode pair p is columns 2p, 2p + 1), so an A
// operand is one 128-bit LDS read per lane. k_gemm_dma moves it with direct
// global-to-LDS loads, three chunks deep; k_gemm loads it into registers and
// writes it to a double buffer with rows padded by 16 bytes. Either way the
// codes of chunk c + 2 are loaded while chunk c computes, and one barrier
// closes a chunk.

// Epilogue: the accumulators (sums of exact fp16 products of integer weights and
// x) are scaled by the row step, the weak columns run as extra 16-deep MFMA
// steps (fp16 weak weights against x gathered at weak_idx), and the result is
// rounded to fp16 (nearest-even).
//
// Block order: the token block varies fastest, so consecutive blocks (which the
// dispatcher deals round-robin to the 8 XCDs) share the rows' codes through the
// MALL, and an XCD's blocks share tokens of x in its L2 when the token blocks
// number 8.
#include <cstdlib>

#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint32_t* q;
    const uint16_t* s;
    const uint8_t* z;
    const int32_t* idx;
    const uint16_t* ww;
    const uint16_t* x;
    uint16_t* y;
    int32_t M, N, K, k;
    int32_t mblocks;  // token blocks (the fastest-varying block index)
};

__device__ __forceinline__ half8_t as_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    uint4 v = make_uint4(a, b, c, d);
    return __builtin_bit_cast(half8_t, v);
}

// FM x FN accumulators per wave, WM x WN waves per block, KH groups per lane
// half per K chunk (a chunk is 2 KH groups = 64 KH columns), WPE waves per SIMD.
template <int FM, int FN, int WM, int WN, int KH, int WPE>
struct Tile {
    static constexpr int NT = 64 * WM * WN;             // threads
    static constexpr int BM = 32 * FM * WM;             // tokens per block
    static constexpr int BN = 32 * FN * WN;             // rows per block
    static constexpr int KG = 2 * KH;                   // groups per chunk
    static constexpr int RB = KG * 64 + 16;             // LDS bytes per staged token (padded)
    static constexpr int XI = (KG * BM + NT - 1) / NT;  // staged group rows per thread
    static constexpr int LDS = 2 * BM * RB + KG * 64;   // double buffer + a spare staging row
};

template <int FM, int FN, int WM, int WN, int KH, int WPE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void k_gemm(GemmArgs a)
{
    using T = Tile<FM, FN, WM, WN, KH, WPE>;
    constexpr int NT = T::NT, BM = T::BM, BN = T::BN, KG = T::KG, RB = T::RB, XI = T::XI;
    extern __shared__ uint4 smem[];
    char* const lds = reinterpret_cast<char*>(smem);

    const int M = a.M, N = a.N, K = a.K, k = a.k;
    const int G = K >> 5;
    const int nchunks = (G + KG - 1) / KG;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int l32 = lane & 31, h = lane >> 5;
    const int m0 = ((int)blockIdx.x % a.mblocks) * BM;
    const int n0 = ((int)blockIdx.x / a.mblocks) * BN;
    const int mv = min(BM, M - m0);  // valid tokens / rows of the block
    const int nv = min(BN, N - n0);

    // x rows and code rows of the block as buffer resources; every offset below
    // is clamped to valid tokens, rows and groups
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x) + (int64_t)m0 * K, (short)0, mv * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(a.q) + (int64_t)n0 * G * 3, (short)0, nv * G * 12, 0x00020000);

    // staging items i = tid + NT t: token i / KG of the block, group i % KG of the chunk
    int xoff[XI];
#pragma unroll
    for (int t = 0; t < XI; t++) {
        const int i = tid + NT * t;
        xoff[t] = min(i / KG, mv - 1) * K * 2;
    }
    // this lane's rows (one per row block f), clamped to the valid rows; their
    // zero points packed one per byte
    const int rbase = wn * 32 * FN + l32;
    auto row_of = [&](int f) { return min(rbase + 32 * f, nv - 1); };
    uint32_t zpk = 0;
#pragma unroll
    for (int f = 0; f < FN; f++)
        zpk |= (uint32_t)a.z[n0 + row_of(f)] << (8 * f);

    // Two chunks in flight: x and codes of chunk c + 2 are loaded while chunk c
    // computes (x into the register set just staged, codes into the set just
    // decoded), so a load has two chunks of MFMA work to arrive in.
    typedef i32x4 XRegs[XI][4];
    typedef u32x3 QRegs[FN][KH];
    auto load_x = [&](int c, XRegs& xg) {
#pragma unroll
        for (int t = 0; t < XI; t++) {
            const int g = min(KG * c + (tid + NT * t) % KG, G - 1);
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                xg[t][q4] = __builtin_amdgcn_raw_buffer_load_b128(xr, xoff[t] + g * 64 + 16 * q4, 0, 0);
        }
    };
    auto load_q = [&](int c, QRegs& cw) {
#pragma unroll
        for (int j = 0; j < KH; j++) {
            const int g = min(KG * c + 2 * j + h, G - 1);
#pragma unroll
            for (int f = 0; f < FN; f++)
                cw[f][j] = __builtin_amdgcn_raw_buffer_load_b96(qr, (row_of(f) * G + g) * 12, 0, 0);
        }
    };
    // x of chunk c into LDS buffer c & 1, in natural column order; a group past the
    // end of K is staged as zeros
    auto stage = [&](int c, const XRegs& xg) {
        char* const buf = lds + (c & 1) * BM * RB;
#pragma unroll
        for (int t = 0; t < XI; t++) {
            const int i = tid + NT * t;
            {
                // threads past the tile's staging items write a spare row instead of branching
                const bool spare = !(KG * BM % NT == 0 || i < KG * BM);
                const bool live = !spare && KG * c + i % KG < G;
                uint32_t pr[16];
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        pr[4 * q4 + e] = live ? (uint32_t)xg[t][q4][e] : 0u;
                uint4* dst = reinterpret_cast<uint4*>(spare ? lds + 2 * BM * RB + (i % KG) * 64
                                                            : buf + (i / KG) * RB + (i % KG) * 64);
#pragma unroll
                for (int q4 = 0; q4 < 4; q4++)
                    dst[q4] = make_uint4(pr[4 * q4], pr[4 * q4 + 1], pr[4 * q4 + 2], pr[4 * q4 + 3]);
            }
        }
    };

    const Magic mg = make_magic();
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int f = 0; f < FN; f++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][f][r] = 0.0f;

    const int arow = (wm * 32 * FM + l32) * RB + h * 64;  // this lane's A operand row
    // Chunk c: x of chunk c + 2 is loaded while the chunk's A operands are read
    // from LDS once and each row block's codes are decoded just before their
    // MFMAs (one 16-register B set live at a time); then the codes of chunk c + 2
    // are loaded into the set just used, x of c + 1 (loaded one step earlier) is
    // staged into the other LDS buffer, and one barrier closes the chunk. All loads are unconditional with
    // clamped addresses, and both steps of a pair always run: a branch would make
    // the compiler wait for every outstanding load at the merge.
    auto step = [&](int c, QRegs& qcur, XRegs& xload, XRegs& xstage) {
        load_x(min(c + 2, nchunks - 1), xload);
        const char* const buf = lds + (c & 1) * BM * RB + arow;
#pragma unroll
        for (int j = 0; j < KH; j++) {
            half8_t av[4][FM];
#pragma unroll
            for (int st = 0; st < 4; st++)
#pragma unroll
                for (int i = 0; i < FM; i++)
                    av[st][i] = __builtin_bit_cast(
                        half8_t, *reinterpret_cast<const uint4*>(buf + i * 32 * RB + 2 * j * 64 + st * 16));
#pragma unroll
            for (int f = 0; f < FN; f++) {
                uint32_t p[16];
                decode_group(qcur[f][j].x, qcur[f][j].y, qcur[f][j].z, mg, make_zero_sub((zpk >> (8 * f)) & 7u), p);
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const half8_t bv = as_h8(p[4 * st], p[4 * st + 1], p[4 * st + 2], p[4 * st + 3]);
#pragma unroll
                    for (int i = 0; i < FM; i++)
                        acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[st][i], bv, acc[i][f], 0, 0, 0);
                }
            }
        }
        load_q(min(c + 2, nchunks - 1), qcur);
        stage(c + 1, xstage);  // zeros past the end of K
        __syncthreads();
    };

    XRegs xa, xb;
    QRegs qa, qb;
    load_x(0, xa);
    load_q(0, qa);
    load_q(min(1, nchunks - 1), qb);
    stage(0, xa);
    load_x(min(1, nchunks - 1), xb);
    __syncthreads();
    // x of chunk c + 1 sits in xb (c even) or xa (c odd), loaded a full step earlier;
    // an odd chunk count runs one extra step on zero-staged x, which adds nothing
    for (int c = 0; c < nchunks; c += 2) {
        step(c, qa, xa, xb);
        step(c + 1, qb, xb, xa);
    }

    // row step, then the weak columns
#pragma unroll
    for (int f = 0; f < FN; f++) {
        const float sc = h2f(a.s[n0 + row_of(f)]);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][f][r] *= sc;
    }
    if (k > 0) {
        int xrow[FM];
#pragma unroll
        for (int i = 0; i < FM; i++)
            xrow[i] = min(wm * 32 * FM + 32 * i + l32, mv - 1) * K;
        for (int cs = 0; cs < k; cs += 16) {
            uint32_t jw[8];
            bool on[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int c = cs + 8 * h + e;
                on[e] = c < k;
                int j = a.idx[min(c, k - 1)];
                jw[e] = (uint32_t)((j >= 0 && j < K) ? j : 0);
            }
            uint32_t bw[FN][4];
#pragma unroll
            for (int f = 0; f < FN; f++) {
                const int64_t row = n0 + min(wn * 32 * FN + 32 * f + l32, nv - 1);
                const uint16_t* wr = a.ww + row * k;
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    const int c = cs + 8 * h + 2 * e2;
                    const uint32_t lo = on[2 * e2] ? wr[c] : 0u;
                    const uint32_t hi = on[2 * e2 + 1] ? wr[c + 1] : 0u;
                    bw[f][e2] = lo | (hi << 16);
                }
            }
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const uint16_t* xm = a.x + (int64_t)m0 * K + xrow[i];
                uint32_t aw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    const uint32_t lo = on[2 * e2] ? xm[jw[2 * e2]] : 0u;
                    const uint32_t hi = on[2 * e2 + 1] ? xm[jw[2 * e2 + 1]] : 0u;
                    aw[e2] = lo | (hi << 16);
                }
                const half8_t av = as_h8(aw[0], aw[1], aw[2], aw[3]);
#pragma unroll
                for (int f = 0; f < FN; f++)
                    acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        av, as_h8(bw[f][0], bw[f][1], bw[f][2], bw[f][3]), acc[i][f], 0, 0, 0);
            }
        }
    }

    // D element r of lane l: token 8 (r / 4) + 4 h + r % 4, row l % 32
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int f = 0; f < FN; f++) {
            const int n = n0 + wn * 32 * FN + 32 * f + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * 32 * FM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M && n < N)
                    a.y[(int64_t)m * N + n] = f2h(acc[i][f][r]);
            }
        }
}

template <int FM, int FN, int WM, int WN, int KH, int WPE>
hipError_t launch_tile(GemmArgs a, hipStream_t s)
{
    using T = Tile<FM, FN, WM, WN, KH, WPE>;
    a.mblocks = (a.M + T::BM - 1) / T::BM;
    const int64_t nblocks = (int64_t)a.mblocks * ((a.N + T::BN - 1) / T::BN);
    if (nblocks > INT32_MAX)
        return hipErrorInvalidValue;
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm<FM, FN, WM, WN, KH, WPE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL((k_gemm<FM, FN, WM, WN, KH, WPE>), dim3((unsigned)nblocks), dim3(T::NT), T::LDS, s, a);
    return hipGetLastError();
}

// Large-M variant: x reaches LDS through gfx950 direct-to-LDS buffer loads (no
// registers, no staging instructions), three chunks deep. A stage is the 64
// columns of a chunk for BM tokens, 128 bytes per token; each thread moves DPW
// 16-byte units per stage, and the unit of (token m, piece c) lands in slot
// c ^ (m & 7) of the token's 128 bytes, so the A-operand reads of a wave (32
// tokens, one piece) hit eight different slots of the bank window. The stages are
// three separate LDS arrays: the compiler then waits only for the loads of the
// stage it reads. Codes run two chunks ahead in three register sets.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

template <int FM, int FN, int WM, int WN>
struct DmaTile {
    static constexpr int NT = 64 * WM * WN;
    static constexpr int BM = 32 * FM * WM;
    static constexpr int BN = 32 * FN * WN;
    static constexpr int STAGE = BM * 128;
    static constexpr int DPW = STAGE / 16 / NT;  // 16-byte units per thread per stage
    static_assert(STAGE % (16 * NT) == 0, "a stage must split evenly over the threads");
};

template <int FM, int FN, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_gemm_dma(GemmArgs a)
{
    using T = DmaTile<FM, FN, WM, WN>;
    constexpr int BM = T::BM, BN = T::BN, STAGE = T::STAGE, DPW = T::DPW;
    __shared__ __attribute__((aligned(1024))) char xs0[STAGE];
    __shared__ __attribute__((aligned(1024))) char xs1[STAGE];
    __shared__ __attribute__((aligned(1024))) char xs2[STAGE];

    const int M = a.M, N = a.N, K = a.K, k = a.k;
    const int G = K >> 5;
    const int nchunks = (G + 1) >> 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM;
    const int l32 = lane & 31, h = lane >> 5;
    const int m0 = ((int)blockIdx.x % a.mblocks) * BM;
    const int n0 = ((int)blockIdx.x / a.mblocks) * BN;
    const int mv = min(BM, M - m0);
    const int nv = min(BN, N - n0);

    // x rows of the block (reads past them return zeros) and code rows
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(a.x) + (int64_t)m0 * K, (short)0, mv * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(a.q) + (int64_t)n0 * G * 3, (short)0, nv * G * 12, 0x00020000);

    // this thread's DMA units: unit u -> token u / 8, slot u % 8, piece slot ^ (token & 7)
    int xsrc[DPW];
#pragma unroll
    for (int t = 0; t < DPW; t++) {
        const int u = (wave * DPW + t) * 64 + lane;
        const int row = u >> 3, piece = (u & 7) ^ (row & 7);
        xsrc[t] = min(row, mv - 1) * K * 2 + piece * 16;
    }
    // the second group of the last chunk lies past K when G is odd: its x pieces
    // (4..7) are read out of range, which returns zeros
    const int last = nchunks - 1;
    const bool odd_tail = (G & 1) != 0;
    int xdead[DPW];
#pragma unroll
    for (int t = 0; t < DPW; t++) {
        const int u = (wave * DPW + t) * 64 + lane;
        xdead[t] = (odd_tail && (((u & 7) ^ ((u >> 3) & 7)) >= 4)) ? 0x40000000 : 0;
    }
    // chunks past the end (the pipeline's tail) are read out of the buffer's
    // range: zeros, and no fetch of the last chunk again
    auto dma = [&](int c, char* stage) {
        const int cc = min(c, last);
        const int dead = c > last ? 0x40000000 : 0;
#pragma unroll
        for (int t = 0; t < DPW; t++)
            dma16(xr, stage + (wave * DPW + t) * 1024, xsrc[t] + cc * 128 + (cc == last ? xdead[t] : 0) + dead);
    };

    const int rbase = wn * 32 * FN + l32;
    auto row_of = [&](int f) { return min(rbase + 32 * f, nv - 1); };
    uint32_t zpk = 0;
#pragma unroll
    for (int f = 0; f < FN; f++)
        zpk |= (uint32_t)a.z[n0 + row_of(f)] << (8 * f);
    typedef u32x3 QRegs[FN];
    auto load_q = [&](int c, QRegs& cw) {
        const int g = min(2 * min(c, nchunks - 1) + h, G - 1);
        const int dead = c >= nchunks ? 0x40000000 : 0;
#pragma unroll
        for (int f = 0; f < FN; f++)
            cw[f] = __builtin_amdgcn_raw_buffer_load_b96(qr, (row_of(f) * G + g) * 12 + dead, 0, 0);
    };

    const Magic mg = make_magic();
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int f = 0; f < FN; f++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][f][r] = 0.0f;

    // this lane's A operand: token row (wm 32 FM + 32 i + l32) * 128, piece h 4 + st
    const int arow = (wm * 32 * FM + l32) * 128;
    int aoff[4];
#pragma unroll
    for (int st = 0; st < 4; st++)
        aoff[st] = ((h * 4 + st) ^ (l32 & 7)) * 16;
    // Chunk c reads stage cur; loads chunk c + 2 into stage nxt2 and code set q2.
    auto step = [&](int c, const char* cur, char* nxt2, const QRegs& qc, QRegs& q2) {
        // this wave's x loads of chunk c are done once at most 2 FN + DPW newer loads
        // remain (codes of c, x and codes of c + 1); after the barrier every wave's
        // are, and every wave has finished reading the stage chunk c + 2 goes to. A
        // plain barrier: a fence here would wait for all x loads in flight.
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * FN + DPW) : "memory");
        dma(c + 2, nxt2);
        load_q(c + 2, q2);
        if (c < nchunks) {  // block-uniform; the steps past the end only keep the pipeline shape
            half8_t av[4][FM];
#pragma unroll
            for (int st = 0; st < 4; st++)
#pragma unroll
                for (int i = 0; i < FM; i++)
                    av[st][i] =
                        __builtin_bit_cast(half8_t, *reinterpret_cast<const uint4*>(cur + arow + i * 32 * 128 + aoff[st]));
#pragma unroll
            for (int f = 0; f < FN; f++) {
                uint32_t p[16];
                decode_group(qc[f].x, qc[f].y, qc[f].z, mg, make_zero_sub((zpk >> (8 * f)) & 7u), p);
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const half8_t bv = as_h8(p[4 * st], p[4 * st + 1], p[4 * st + 2], p[4 * st + 3]);
#pragma unroll
                    for (int i = 0; i < FM; i++)
                        acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[st][i], bv, acc[i][f], 0, 0, 0);
                }
            }
        }
    };

    QRegs qa, qb, qc3;
    // the prologue issues x and codes chunk by chunk, in the order the steps
    // do, so the waits inserted for the code registers count the same loads on
    // the first pass through the loop as on the others
    dma(0, xs0);
    load_q(0, qa);
    asm volatile("" ::: "memory");
    dma(1, xs1);
    load_q(1, qb);
    asm volatile("" ::: "memory");
    for (int c = 0; c < nchunks; c += 3) {
        step(c, xs0, xs2, qa, qc3);
        step(c + 1, xs1, xs0, qb, qa);
        step(c + 2, xs2, xs1, qc3, qb);
    }
    // the last steps' x loads (duplicates of the last chunk) may still be in
    // flight: none may write LDS after the block has ended (waited here, so the
    // block need not wait for its output stores)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // row step, then the weak columns
#pragma unroll
    for (int f = 0; f < FN; f++) {
        const float sc = h2f(a.s[n0 + row_of(f)]);
#pragma unroll
        for (int i = 0; i < FM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][f][r] *= sc;
    }
    if (k > 0) {
        int xrow[FM];
#pragma unroll
        for (int i = 0; i < FM; i++)
            xrow[i] = min(wm * 32 * FM + 32 * i + l32, mv - 1) * K;
        for (int cs = 0; cs < k; cs += 16) {
            uint32_t jw[8];
            bool on[8];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const int c = cs + 8 * h + e;
                on[e] = c < k;
                int j = a.idx[min(c, k - 1)];
                jw[e] = (uint32_t)((j >= 0 && j < K) ? j : 0);
            }
#pragma unroll
            for (int i = 0; i < FM; i++) {
                const uint16_t* xm = a.x + (int64_t)m0 * K + xrow[i];
                uint32_t aw[4];
#pragma unroll
                for (int e2 = 0; e2 < 4; e2++) {
                    const uint32_t lo = on[2 * e2] ? xm[jw[2 * e2]] : 0u;
                    const uint32_t hi = on[2 * e2 + 1] ? xm[jw[2 * e2 + 1]] : 0u;
                    aw[e2] = lo | (hi << 16);
                }
                const half8_t av = as_h8(aw[0], aw[1], aw[2], aw[3]);
#pragma unroll
                for (int f = 0; f < FN; f++) {
                    const uint16_t* wr = a.ww + (int64_t)(n0 + row_of(f)) * k;
                    uint32_t bw[4];
#pragma unroll
                    for (int e2 = 0; e2 < 4; e2++) {
                        const int c = cs + 8 * h + 2 * e2;
                        const uint32_t lo = on[2 * e2] ? wr[c] : 0u;
                        const uint32_t hi = on[2 * e2 + 1] ? wr[c + 1] : 0u;
                        bw[e2] = lo | (hi << 16);
                    }
                    acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, as_h8(bw[0], bw[1], bw[2], bw[3]),
                                                                       acc[i][f], 0, 0, 0);
                }
            }
        }
    }

    // D element r of lane l: token 8 (r / 4) + 4 h + r % 4, row l % 32
#pragma unroll
    for (int i = 0; i < FM; i++)
#pragma unroll
        for (int f = 0; f < FN; f++) {
            const int n = n0 + wn * 32 * FN + 32 * f + l32;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + wm * 32 * FM + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M && n < N)
                    a.y[(int64_t)m * N + n] = f2h(acc[i][f][r]);
            }
        }
}

template <int FM, int FN, int WM, int WN>
hipError_t launch_dma(GemmArgs a, hipStream_t s)
{
    using T = DmaTile<FM, FN, WM, WN>;
    a.mblocks = (a.M + T::BM - 1) / T::BM;
    const int64_t nblocks = (int64_t)a.mblocks * ((a.N + T::BN - 1) / T::BN);
    if (nblocks > INT32_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_gemm_dma<FM, FN, WM, WN>), dim3((unsigned)nblocks), dim3(T::NT), 0, s, a);
    return hipGetLastError();
}

int64_t env_min_m()
{
    const char* e = std::getenv("OWQ_GEMM_MIN_M");
    if (e && *e) {
        const long long v = std::atoll(e);
        if (v >= 1)
            return v;
    }
    return 17;
}

}  // namespace

int64_t gemm_min_m()
{
    static const int64_t v = env_min_m();
    return v;
}

hipError_t launch_gemm(const LinearDesc& d, int64_t M, hipStream_t s)
{
    GemmArgs a;
    a.q = d.q;
    a.s = d.s;
    a.z = d.z;
    a.idx = d.idx;
    a.ww = d.ww;
    a.x = d.x;
    a.y = d.y;
    a.M = (int32_t)M;
    a.N = (int32_t)d.N;
    a.K = (int32_t)d.K;
    a.k = d.k;
    a.mblocks = 1;
    if (M >= 128)
        return launch_dma<2, 4, 2, 2>(a, s);     // 128 tokens x 256 rows, 4 waves of 64 x 128
    return launch_tile<1, 2, 1, 4, 1, 2>(a, s);  // 32 tokens x 256 rows, 4 waves of 32 x 64
}

}  // namespace owq
