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
// the groups 4 u + l / 16 (u < U) of each K chunk of 4 U groups (the codes are
// loaded as whole lines and regrouped through LDS, see load_q); the 16 decode
// pairs of a group feed four MFMA steps (pairs 4t .. 4t + 3 in step t). Decode pair p is columns (2p, 2p + 1) (the slot layout of the codes),
// so x is staged as it is stored: the block's x chunk sits in LDS as
// [token][group][32 values] and an A operand is one 128-bit LDS read per lane.
// The K reduction happens inside the accumulators: no cross-lane reduction.
//
// Pipeline: x by direct-to-LDS loads into D + 1 stages and codes into D + 1
// register sets, D chunks ahead of the one computed (D = 1 or 2), one barrier
// per chunk.
// A block is W row waves (16 W rows of one layer) times S groups that split K;
// one launch covers a batch of layers of any shapes.
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


__device__ __forceinline__ half8_t h8_of(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(half8_t, make_uint4(a, b, c, d));
}

// U groups per lane per chunk; MC = largest token count of the instance.
template <int U, int MC>
struct MfvShape {
    static constexpr int GC = 4 * U;             // groups per chunk
    static constexpr int RS = GC * 64 + 16;      // LDS bytes per staged token (padded)
    static constexpr int STAGE = MC * RS;        // one x stage
    static constexpr int PT = GC / 16;           // 1 KB x loads per token and chunk
    static constexpr int DPW = MC * PT / 4;      // x loads per wave and chunk
    static constexpr int CRS = GC * 12 + 16;     // LDS bytes per row of a wave's code chunk (padded)
    static constexpr int CQ = GC * 12 / 16;      // 16-byte pieces of a row's code chunk
    static constexpr int CL = 16 * CQ / 64;      // code loads per lane and chunk
    static_assert(GC % 16 == 0 && (MC * PT) % 4 == 0, "x loads must split evenly over the waves");
    static_assert((16 * CQ) % 64 == 0 && CRS % 16 == 0, "code pieces must split evenly over the lanes");
};

__device__ __forceinline__ void dma_x(__amdgpu_buffer_rsrc_t r, char* lds, int voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}

// S groups of W wavefronts split K: group kg walks chunks [kg P, kg P + P) of
// the layer (P = ceil(chunks / S)) with x stages of its own, all groups in step
// (one block barrier per chunk); at the end groups 1 .. S - 1 hand their
// accumulators to group 0 through LDS. This cuts the chain of dependent chunks
// of a block by S, so the blocks of long-row layers do not run on alone after
// the others have finished.
template <int U, int MC, int W, int S, int D>
__global__ __launch_bounds__(64 * W * S) void k_mfv(MfvBatch b, int M)
{
    using SH = MfvShape<U, MC>;
    constexpr int GC = SH::GC, RS = SH::RS, STAGE = SH::STAGE, PT = SH::PT;
    constexpr int DPW = MC * PT / W;  // x loads per wave and chunk
    // the codes are read once per launch; with 8- and 16-token x stages
    // non-temporal code loads (cache policy "nt") were 5-7 % faster (1-4 % slower
    // at M <= 4). A row's code chunk is GC * 12 bytes: with U = 4 that is 192
    // bytes, 1.5 cache lines, so two chunks share a line, and without a cached
    // copy the shared line is fetched again for the second chunk (1.39x of the
    // algorithmic bytes at M = 16, 1.16x with default loads); with U = 8 (the
    // 8-token instance) a chunk is 384 bytes, three whole lines of rows whose
    // length is a multiple of 128 bytes
    constexpr int kCodePolicy = MC >= 8 ? 2 : 0;
    static_assert((MC * PT) % W == 0, "x loads must split evenly over the waves");
    constexpr int CRS = SH::CRS, CQ = SH::CQ, CL = SH::CL;
    // D + 1 x stages per K group (chunks run D ahead), each its own array
    __shared__ __attribute__((aligned(1024))) char xs0[S][STAGE];
    __shared__ __attribute__((aligned(1024))) char xs1[S][STAGE];
    __shared__ __attribute__((aligned(1024))) char xs2[D == 2 ? S : 1][D == 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) char cs[W * S][16 * CRS];  // each wave's code chunk
    static_assert(S == 1 || (S - 1) * W * 64 * 16 <= STAGE * S, "partial sums must fit in one stage set");

    int li = 0;
    for (int l = 1; l < b.count; l++)
        if ((int)blockIdx.x >= b.L[l].block0)
            li = l;
    const MfvLayer& L = b.L[li];
    const int N = L.N, K = L.K, k = L.k;
    const int G = K >> 5;
    const int nch = (G + GC - 1) / GC;
    const int per = (nch + S - 1) / S;  // chunks per K group
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wid % W, kg = wid / W;  // row wave in the block, K group
    const int c0 = kg * per, c1 = min(nch, c0 + per);  // this group's chunks
    const int l16 = lane & 15, qd = lane >> 4;
    const int brow = ((int)blockIdx.x - L.block0) * 16 * W;
    const int nb = min(N - brow, 16 * W);  // valid rows of the block
    const int rloc = min(wave * 16 + l16, nb - 1);  // this lane's row in the block (clamped)

    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(L.q) + (int64_t)brow * G * 3, (short)0, nb * G * 12, 0x00020000);
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(L.x), (short)0, M * K * 2, 0x00020000);

    // x of chunk c goes to LDS by direct-to-LDS loads: load t of this wave moves
    // 1 KB (16 groups) of token m = qi / PT, qi = wave DPW + t, to stage offset
    // m RS + (qi % PT) KB; lanes 4 apart take consecutive groups. Groups past K,
    // and chunks past the group's range, are read out of the buffer's range,
    // which gives zeros; tokens past M repeat the last token (their A rows are
    // never read).
    auto dma = [&](int c, char* stage) {
        const int cc = min(c, c1 - 1);
        const int dead = c >= c1 ? 0x40000000 : 0;
#pragma unroll
        for (int t = 0; t < DPW; t++) {
            const int qi = wave * DPW + t;
            const int m = qi / PT, part = qi % PT;
            const int g = cc * GC + part * 16 + (lane >> 2);
            const int off = (min(m, M - 1) * K + g * 32) * 2 + (lane & 3) * 16;
            dma_x(xr, stage + m * RS + part * 1024, off + (g >= G ? 0x40000000 : dead));
        }
    };
    // Codes: the wave's 16 rows x GC groups of a chunk are loaded as consecutive
    // 16-byte pieces (piece p = 64 i + lane: row p / CQ, bytes 16 (p % CQ) of the
    // row's chunk), so each load instruction reads whole lines; the MFMA layout
    // wants group 4 u + l / 16 of row l % 16 in lane l, so the pieces go through
    // the wave's own LDS rows (padded to CRS bytes: the group reads of a wave
    // then hit distinct banks). Rows past the block and groups past K read zeros
    // or the next row; their x is zero.
    typedef uint4 QRegs[CL];
    // chunks past the group's range (the pipeline's tail) are read out of the
    // buffer's range, which returns zeros and fetches nothing: clamped to the
    // last chunk they would read it again, from memory with non-temporal loads
    auto load_q = [&](int c, QRegs& cw) {
        const int cc = min(c, c1 - 1);
        const int dead = c >= c1 ? 0x40000000 : 0;
#pragma unroll
        for (int i = 0; i < CL; i++) {
            const int pc = 64 * i + lane;
            const int r = pc / CQ, o = (pc % CQ) * 16;
            cw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                  qr, ((wave * 16 + r) * G + cc * GC) * 12 + o + dead, 0, kCodePolicy));
        }
    };
    char* const crow = cs[wid];

    const float sc = h2f(L.s[brow + rloc]);
    const ZeroSub zs = make_zero_sub((uint32_t)L.z[brow + rloc]);
    const Magic mg = make_magic();
    // one accumulator per group slot u: the MFMAs of different groups do not
    // wait for each other's results
    f32x4 accu[U];
#pragma unroll
    for (int u = 0; u < U; u++)
        accu[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // this lane's A operand: token min(l16, M - 1), groups 4 u + qd of the chunk
    const int arow = min(l16, M - 1) * RS + qd * 64;
    // Chunk c reads stage cur and codes qc; it loads x and codes of chunk c + D
    // into stage nxt and set qn first.
    auto step = [&](int c, const char* cur, char* nxt, const QRegs& qc, QRegs& qn) {
        // this wave's x loads of chunk c are done once at most D CL + (D - 1) DPW
        // newer loads remain (codes of c, x and codes of c + 1 .. c + D - 1);
        // after the barrier every wave's are, and every wave is done with the
        // stage chunk c + D goes to
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(D * CL + (D - 1) * DPW) : "memory");
        dma(c + D, nxt);
        load_q(c + D, qn);
        if (c < c1) {  // wave-uniform; the steps past the end only keep the pipeline shape
#pragma unroll
            for (int i = 0; i < CL; i++) {
                const int pc = 64 * i + lane;
                *reinterpret_cast<uint4*>(crow + (pc / CQ) * CRS + (pc % CQ) * 16) = qc[i];
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                const uint32_t* gw = reinterpret_cast<const uint32_t*>(crow + l16 * CRS + (4 * u + qd) * 12);
                uint32_t p[16];
                decode_group(gw[0], gw[1], gw[2], mg, zs, p);
#pragma unroll
                for (int st = 0; st < 4; st++) {
                    const half8_t av = __builtin_bit_cast(
                        half8_t, *reinterpret_cast<const uint4*>(cur + arow + 4 * u * 64 + st * 16));
                    accu[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        av, h8_of(p[4 * st], p[4 * st + 1], p[4 * st + 2], p[4 * st + 3]), accu[u], 0, 0, 0);
                }
            }
        }
    };

    QRegs qa, qb, qc3;
    // the prologue issues x and codes chunk by chunk, in the order the steps
    // do, so the waits inserted for the code registers count the same loads on
    // the first pass through the loop as on the others
    if constexpr (D == 2) {
        dma(c0, xs0[kg]);
        load_q(c0, qa);
        asm volatile("" ::: "memory");
        dma(c0 + 1, xs1[kg]);
        load_q(c0 + 1, qb);
        asm volatile("" ::: "memory");
        for (int c = c0; c < c0 + per; c += 3) {  // the same trip count in every group
            step(c, xs0[kg], xs2[kg], qa, qc3);
            step(c + 1, xs1[kg], xs0[kg], qb, qa);
            step(c + 2, xs2[kg], xs1[kg], qc3, qb);
        }
    } else {
        dma(c0, xs0[kg]);
        load_q(c0, qa);
        asm volatile("" ::: "memory");
        for (int c = c0; c < c0 + per; c += 2) {
            step(c, xs0[kg], xs1[kg], qa, qb);
            step(c + 1, xs1[kg], xs0[kg], qb, qa);
        }
    }
    // the last steps' x loads may still be in flight: none may write LDS after
    // this point (the stages are reused below, and the block may end)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4 acc = accu[0];
#pragma unroll
    for (int u = 1; u < U; u++)
        acc += accu[u];

    if constexpr (S > 1) {  // K groups 1 .. S - 1 hand their sums to group 0
        f32x4* part = reinterpret_cast<f32x4*>(&xs0[0][0]);
        __syncthreads();
        if (kg > 0)
            part[((kg - 1) * W + wave) * 64 + lane] = acc;
        __syncthreads();
        if (kg > 0)
            return;
#pragma unroll
        for (int g2 = 1; g2 < S; g2++)
            acc += part[((g2 - 1) * W + wave) * 64 + lane];
    }

    // row step, then the weak columns: B = w_weak[row][cs + 8 qd + e], A = x[token][idx[...]]
#pragma unroll
    for (int r = 0; r < 4; r++)
        acc[r] *= sc;
    if (k > 0) {
        const uint16_t* wr = L.ww + (int64_t)(brow + rloc) * k;
        const uint16_t* xm = L.x + (int64_t)min(l16, M - 1) * K;
        for (int cs2 = 0; cs2 < k; cs2 += 32) {
            uint32_t bw[4], aw[4];
#pragma unroll
            for (int e2 = 0; e2 < 4; e2++) {
                uint32_t wv[2], xv[2];
#pragma unroll
                for (int h = 0; h < 2; h++) {
                    const int c = cs2 + 8 * qd + 2 * e2 + h;
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

template <int U, int MC, int W, int S, int D>
hipError_t launch_shape(const MfvBatch& b, int nblocks, int M, hipStream_t s)
{
    hipLaunchKernelGGL((k_mfv<U, MC, W, S, D>), dim3(nblocks), dim3(64 * W * S), 0, s, b, M);
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
    return M > kVectorDecodeMaxM;
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
    // up to 4 tokens: blocks of 2 row waves x 2 K groups (the 4096 x 11008
    // blocks then finish with the rest); more tokens: 4 row waves over the whole
    // row (the 8- and 16-token x stages leave LDS for no second K group)
    const int W = M <= 4 ? 2 : 4;
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
        nblocks += (int)((dl.N + 16 * W - 1) / (16 * W));
    }
    // x of up to 4 tokens: one chunk ahead (two stages: five waves per SIMD
    // instead of four, 6 % faster); 16 tokens: two ahead (one ahead leaves more
    // waves but was 3-6 % slower)
    if (M <= 4)
        return launch_shape<4, 4, 2, 2, 1>(b, nblocks, M, s);
    // 5 to 8 tokens: 32-group chunks (whole cache lines of codes, see
    // kCodePolicy), two chunks ahead; 16-token stages of 32 groups would leave
    // one block per CU (32.7 against 32.2 us at M = 8 with 16-group chunks, 39 us
    // at M = 16 with one chunk ahead)
    if (M <= 8)
        return launch_shape<8, 8, 4, 1, 2>(b, nblocks, M, s);
    return launch_shape<4, 16, 4, 1, 2>(b, nblocks, M, s);
}

}  // namespace owq
