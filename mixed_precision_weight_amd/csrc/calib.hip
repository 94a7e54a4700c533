// calib.hip -- calibration kernels: Hessian diagonal, row fit, column RTN errors,
// column scores (gfx950).
//
// The layer-wise error ||W X^T - W^ X^T||^2 splits into one quadratic error per
// output row, all sharing the Hessian H = 2 X^T X ([PL] "Error Decomposition",
// "Error Analysis", paper p.3 and appendix section 1 p.10). Column sensitivity
// is the Hessian diagonal element times the squared perturbation norm of the
// column ([PL] "Weak-column selection", paper p.4):
//     lambda_j = 2 sum_t X[t][j]^2,   e_j = sum_i dW_ij^2,   score_j = lambda_j e_j,
// with dW the round-to-nearest error of a full-row min-max fit.
// [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models".
//
// Both sums are column reductions of an fp16 [R][K] matrix streamed from HBM,
// and e_j needs each row's fit (min and max over the whole row) first.
//
// W is read once: a block of the fused form owns whole rows, 8 (or 16) fp16
// columns per lane in 16-byte words, G rows at a time with the next G rows'
// loads in flight. Each row's min and max are reduced across the block (DPP
// within a wave, one LDS exchange and one barrier per G rows), lane g of every
// wave turns row g's range into (step, zero point), readlane hands them to the
// whole wave, and every lane adds the squared RTN errors of its own columns to
// fp64 accumulators that stay in registers across the block's rows: no
// cross-lane sum, one [K] partial row per block. Rows wider than 4096 words
// (K > 32768) keep the two-pass form: one wave per row fit, then column tiles
// of the errors.
//
// X: a block owns a 64-column tile of one row slice. Lane (wave w, lane l) reads
// 8 columns (16 B) at column 8*(l%8) of rows w*8 + l/8 + 8*nwaves*t, so each
// wave instruction reads 8 full 128-byte lines; squares accumulate in fp64, the
// 8 row phases of a wave are combined by a fixed butterfly, the waves by a
// fixed-order LDS sum.
//
// A last launch sums the partial rows of every linear in a fixed order: results
// are bitwise deterministic.
//
// Built with -ffp-contract=off: the quantiser steps are single IEEE operations.
#include <algorithm>
#include <mutex>
#include <vector>

#include "owq_device.h"
#include "owq_launch.h"

// Library-owned calibration workspace for callers that cannot allocate
// (owq_calibrate_score_noalloc). One copy per GPU, created when the library's
// code object is loaded on that GPU and held until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device (calib_scratch).
static __device__ __align__(256) unsigned char scratch[owq::kCalibScratchBytes];

namespace owq {

namespace {

constexpr int kTileCols = 64;   // columns per X (or two-pass error) tile
constexpr int kUnroll = 4;      // rows in flight per lane in a tile
constexpr int kMaxWaves = 16;   // waves per block
constexpr int kWPolicy = 2;     // buffer-load cache policy of the W rows: non-temporal (read once)
constexpr bool kXNonTemporal = false;  // X tile loads non-temporal

struct SqElem {  // x^2 (exact in fp32 for fp16 x)
    struct Row {};
    __device__ __forceinline__ Row load_row(int64_t) const { return Row{}; }
    __device__ __forceinline__ float val(const Row&, uint16_t h) const
    {
        float v = h2f(h);
        return v * v;
    }
    static constexpr bool kSquared = true;
};

// The residual against the (possibly clamped) grid point, exact: every weight
// lies inside the row's full-row fit range, so |w / s| <= 8 and the product of
// the offset and the 11-bit step has at most 14 bits. The rounded quotient
// t = rint(w rs) is rint(w / s) except possibly at an exact half-integer (see
// rint_quotient), where both neighbours leave |residual| = s / 2, and the clamp
// to the code range maps an out-of-range neighbour onto the in-range one; the
// squared residual is therefore the same as with the tie rounded to even.
__device__ __forceinline__ float rtn_residual(float w, float s, float rs, float lo, float hi)
{
    const float q = __builtin_amdgcn_fmed3f(rintf(w * rs), lo, hi);
    return __builtin_fmaf(-q, s, w);
}

struct ErrElem {  // dW = w - s (q - z), exact in fp32; squared in fp64 by the caller
    const uint16_t* s16;
    const uint8_t* z;
    typedef RtnRow Row;
    __device__ __forceinline__ Row load_row(int64_t r) const { return make_rtn_row(h2f(s16[r]), z[r]); }
    __device__ __forceinline__ float val(const Row& rw, uint16_t h) const
    {
        return rtn_residual(h2f(h), rw.s, rw.rs, rw.lo, rw.hi);
    }
    static constexpr bool kSquared = false;
};

// Column sums of one 64-column tile over one row slice, into partial[slice][.]
template <class Elem>
__device__ __forceinline__ void colsum_tile(const uint16_t* __restrict__ A, int64_t R, int64_t K,
                                            int64_t rows_per_slice, double* __restrict__ partial, Elem elem,
                                            int64_t tile, int64_t slice, double (&red)[kMaxWaves][kTileCols])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int phases = nwaves * 8;
    const int cc = lane & 7;
    const int phase = wave * 8 + (lane >> 3);
    const int64_t col = tile * kTileCols + cc * 8;
    const bool active = col < K;
    const int64_t colc = active ? col : 0;  // loads stay in bounds; inactive lanes add nothing
    const int64_t r0 = slice * rows_per_slice;
    const int64_t r1 = min(R, r0 + rows_per_slice);

    double acc[8];
#pragma unroll
    for (int c = 0; c < 8; c++)
        acc[c] = 0.0;

    // every load of an unrolled step is issued before the first use: rows are
    // clamped to the slice instead of branched around
    for (int64_t rb = r0 + phase; rb < r1; rb += (int64_t)phases * kUnroll) {
        uint4 v[kUnroll];
        typename Elem::Row rw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t r = min(rb + (int64_t)u * phases, r1 - 1);
            if constexpr (kXNonTemporal) {
                typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
                v[u] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(A + r * K + colc)));
            } else {
                v[u] = *reinterpret_cast<const uint4*>(A + r * K + colc);
            }
            rw[u] = elem.load_row(r);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            if (!(active && rb + (int64_t)u * phases < r1))
                continue;
            uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int c = 0; c < 8; c++) {
                uint16_t h = (uint16_t)(w[c >> 1] >> (16 * (c & 1)));
                float e = elem.val(rw[u], h);
                if (Elem::kSquared)
                    acc[c] += (double)e;
                else  // e^2 is exact in fp64, so the fused form rounds like mul + add
                    acc[c] = __builtin_fma((double)e, (double)e, acc[c]);
            }
        }
    }
    // combine the 8 row phases of this wave (lanes differing in bits 3..5)
#pragma unroll
    for (int c = 0; c < 8; c++) {
        acc[c] += shfl_xor_f64(acc[c], 8);
        acc[c] += shfl_xor_f64(acc[c], 16);
        acc[c] += shfl_xor_f64(acc[c], 32);
    }
    if (lane < 8) {
#pragma unroll
        for (int c = 0; c < 8; c++)
            red[wave][lane * 8 + c] = acc[c];
    }
    __syncthreads();
    if (threadIdx.x < kTileCols) {
        int64_t j = tile * kTileCols + threadIdx.x;
        if (j < K) {
            double t = red[0][threadIdx.x];
            for (int w = 1; w < nwaves; w++)
                t += red[w][threadIdx.x];
            partial[slice * K + j] = t;
        }
    }
}

// Two-pass form: one wave per row, min/max over all K columns -> (fp16 step,
// zero point).
__device__ __forceinline__ void rowfit_rows(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                            uint16_t* __restrict__ s16, uint8_t* __restrict__ z, int64_t blk)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = blk * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (row >= N)
        return;
    const uint4* p = reinterpret_cast<const uint4*>(W + row * K);
    const int64_t n16 = K / 8;  // 16-byte words of the row
    float lo = 0.0f, hi = 0.0f;
    // 8 words per lane in flight; clamped reloads of the last word change no min/max
    for (int64_t c0 = lane; c0 < n16; c0 += 64 * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            v[u] = p[min(c0 + 64 * u, n16 - 1)];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int i = 0; i < 8; i++) {
                float f = h2f((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
                lo = fminf(lo, f);
                hi = fmaxf(hi, f);
            }
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    if (lane == 0) {
        uint16_t s;
        int zz;
        qparams_from_range(lo, hi, s, zz);
        s16[row] = s;
        z[row] = (uint8_t)zz;
    }
}

// round(w s) for the fp16 in the low (HI = 0) or high (HI = 1) half of h2 and
// an fp32 s: one v_fma_mix_f32 with a zero addend (the exact product rounded
// once, as the fp32 product of the widened value; only a zero's sign may
// differ, which no caller looks at)
template <int HI>
__device__ __forceinline__ float mul_h(uint32_t h2, float s)
{
    float r;
    if constexpr (HI)
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(s));
    else
        asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(s));
    return r;
}

__device__ __forceinline__ uint32_t h2max(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_maximum(__builtin_bit_cast(half2_t, a),
                                                                      __builtin_bit_cast(half2_t, b)));
}

// DPP move: every lane has a source (quad permutes, row rotations)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_all(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// DPP move into the rows of ROWS only; the other lanes keep their own value
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_rows(uint32_t v)
{
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROWS, 0xf, false);
}

// Both halves' maxima over the wave's 64 lanes (exact), as a wave-uniform value.
__device__ __forceinline__ uint32_t wave_h2max(uint32_t v)
{
    v = h2max(v, dpp_all<0xb1>(v));          // quad_perm [1,0,3,2]
    v = h2max(v, dpp_all<0x4e>(v));          // quad_perm [2,3,0,1]
    v = h2max(v, dpp_all<0x124>(v));         // row_ror:4
    v = h2max(v, dpp_all<0x128>(v));         // row_ror:8
    v = h2max(v, dpp_rows<0x142, 0xa>(v));   // row_bcast:15 into rows 1, 3
    v = h2max(v, dpp_rows<0x143, 0xc>(v));   // row_bcast:31 into rows 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Fused form: rows [r0, r1) of W, every column; part = this block's [K] row of
// column error sums, in row order. Lane slot u holds the 16-byte word
// tid + blockDim.x u of a row. Loads go through a buffer resource over the
// block's rows: slots past the row and rows past the block (also the
// prefetch's tail) are read out of range, which returns zeros and fetches
// nothing; a zero changes no min or max (the fit range contains 0), and those
// slots and rows are never accumulated or stored. A row's range travels as the
// fp16 pair (-min, max), reduced with one packed max.
template <int WPL, int G, int D>
__device__ __forceinline__ void fit_err_rows(const uint16_t* __restrict__ W, int64_t K, int64_t r0, int64_t r1,
                                             double* __restrict__ part, uint32_t (&mm)[3][G][kMaxWaves])
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwaves = blockDim.x >> 6;
    const int64_t nw = K >> 3;
    constexpr uint32_t kDead = 0x40000000u;
    uint32_t off[WPL];  // byte offset of the lane's word in a row, or out of range
    bool act[WPL];
#pragma unroll
    for (int u = 0; u < WPL; u++) {
        const int64_t wd = tid + (int64_t)blockDim.x * u;
        act[u] = wd < nw;
        off[u] = act[u] ? 16u * (uint32_t)wd : kDead;
    }
    const uint32_t row_bytes = (uint32_t)(2 * K);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W + r0 * K), (short)0, (int)((r1 - r0) * row_bytes), 0x00020000);
    double acc[WPL][8];
#pragma unroll
    for (int u = 0; u < WPL; u++)
#pragma unroll
        for (int c = 0; c < 8; c++)
            acc[u][c] = 0.0;

    typedef uint4 Rows[G][WPL];
    auto load = [&](Rows& d, int64_t rb) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            const uint32_t ro = (uint32_t)(rb + g - r0) * row_bytes;  // past r1: out of range
#pragma unroll
            for (int u = 0; u < WPL; u++)
                d[g][u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, ro + off[u], 0, kWPolicy));
        }
    };
    // rows rb .. rb + G - 1 held in v; the loads of rows rb + D G .. go to vn first
    auto step = [&](int64_t rb, const Rows& v, Rows& vn, int buf) {
        load(vn, rb + D * G);
#pragma unroll
        for (int g = 0; g < G; g++) {
            uint32_t nmn = 0, mx = 0;  // (min, max) pairs of the lane's columns, from 0
#pragma unroll
            for (int u = 0; u < WPL; u++) {
                const half2_t a = __builtin_bit_cast(half2_t, v[g][u].x), b = __builtin_bit_cast(half2_t, v[g][u].y);
                const half2_t c = __builtin_bit_cast(half2_t, v[g][u].z), d = __builtin_bit_cast(half2_t, v[g][u].w);
                half2_t m0 = __builtin_bit_cast(half2_t, nmn), m1 = __builtin_bit_cast(half2_t, mx);
                m0 = __builtin_elementwise_minimum(__builtin_elementwise_minimum(m0, a), b);
                m0 = __builtin_elementwise_minimum(__builtin_elementwise_minimum(m0, c), d);
                m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m1, a), b);
                m1 = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m1, c), d);
                nmn = __builtin_bit_cast(uint32_t, m0);
                mx = __builtin_bit_cast(uint32_t, m1);
            }
            const half2_t m0 = __builtin_bit_cast(half2_t, nmn), m1 = __builtin_bit_cast(half2_t, mx);
            const half2_t pr = {(_Float16)(-__builtin_elementwise_minimum(m0[0], m0[1])),
                                __builtin_elementwise_maximum(m1[0], m1[1])};
            const uint32_t r = wave_h2max(__builtin_bit_cast(uint32_t, pr));
            if (lane == 0)
                mm[buf][g][wave] = r;
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        // lane g of every wave fits row g
        float fs = 1.0f, frs = 1.0f, flo = 0.0f, fhi = 0.0f;
        if (lane < G) {
            uint32_t m = 0;
            for (int w = 0; w < nwaves; w++)
                m = h2max(m, mm[buf][lane][w]);
            const half2_t h = __builtin_bit_cast(half2_t, m);
            uint16_t s16;
            int z;
            qparams_from_range(-(float)h[0], (float)h[1], s16, z);
            const RtnRow rr = make_rtn_row(h2f(s16), z);
            fs = rr.s;
            frs = rr.rs;
            flo = rr.lo;
            fhi = rr.hi;
        }
#pragma unroll
        for (int g = 0; g < G; g++) {
            if (rb + g >= r1)  // block-uniform
                break;
            const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fs), g));
            const float rs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, frs), g));
            const float qlo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, flo), g));
            const float qhi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fhi), g));
#pragma unroll
            for (int u = 0; u < WPL; u++) {
                const uint32_t w4[4] = {v[g][u].x, v[g][u].y, v[g][u].z, v[g][u].w};
#pragma unroll
                for (int c = 0; c < 8; c++) {
                    const uint32_t h2 = w4[c >> 1];
                    const float t = (c & 1) ? mul_h<1>(h2, rs) : mul_h<0>(h2, rs);
                    const float q = __builtin_amdgcn_fmed3f(rintf(t), qlo, qhi);
                    const float e = __builtin_fmaf(-q, s, h2f((uint16_t)(h2 >> (16 * (c & 1)))));
                    acc[u][c] = __builtin_fma((double)e, (double)e, acc[u][c]);
                }
            }
        }
    };
    if constexpr (D == 1) {
        Rows va, vb;
        load(va, r0);
        for (int64_t rb = r0; rb < r1; rb += 2 * G) {  // the two row buffers take turns
            step(rb, va, vb, 0);
            if (rb + G >= r1)
                break;
            step(rb + G, vb, va, 1);
        }
    } else {  // D == 2: three row buffers, two groups in flight
        Rows va, vb, vc;
        load(va, r0);
        load(vb, r0 + G);
        for (int64_t rb = r0; rb < r1; rb += 3 * G) {
            step(rb, va, vc, 0);  // consecutive steps use different range slots
            if (rb + G >= r1)
                break;
            step(rb + G, vb, va, 1);
            if (rb + 2 * G >= r1)
                break;
            step(rb + 2 * G, vc, vb, 2);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's out-of-range loads
#pragma unroll
    for (int u = 0; u < WPL; u++) {
        if (!act[u])
            continue;
        double2* p = reinterpret_cast<double2*>(part + off[u] / 2);
#pragma unroll
        for (int c = 0; c < 4; c++)
            p[c] = make_double2(acc[u][2 * c], acc[u][2 * c + 1]);
    }
}

// ---------------------------------------------------------------------------
// One launch holds up to kCalibMaxLayers linears, and three kinds of blocks, in
// this order: [wb[l], wb[l+1]) are linear l's W blocks (the long ones start
// first), then [fb[l], fb[l+1]) its final-sum blocks, then [xb[l], xb[l+1]) its
// X blocks. A launch of one group of linears also carries the final sums of
// the group before it, whose partial sums the previous launch wrote.
constexpr int kCalibMaxLayers = 16;
constexpr int kCalibChunk = kCalibMaxLayers / 2;  // linears whose sums one launch computes

struct CalibLayer {
    const uint16_t* W;
    const uint16_t* X;
    double* px;
    double* pw;
    uint16_t* s16;
    uint8_t* z;
    double* lambda;
    double* score;
    int64_t N, K, T, rows_x, rows_w, sx, sw, tiles;
};

struct CalibLaunch {
    CalibLayer L[kCalibMaxLayers];
    int32_t wb[kCalibMaxLayers + 1];
    int32_t fb[kCalibMaxLayers + 1];
    int32_t xb[kCalibMaxLayers + 1];
    int32_t count;
};

__device__ __forceinline__ int layer_of(const int32_t* b0, int count, int64_t b)
{
    int l = 0;
    while (l + 1 < count && b >= b0[l + 1])
        l++;
    return l;
}

// Final sums: kFinCols columns per block, kFinParts partial sums per column.
constexpr int kFinCols = 16;
constexpr int kFinParts = 64;

// LDS of every role: the tile sums' [kMaxWaves][kTileCols] doubles and the final
// sums' [2][kFinParts][kFinCols]
constexpr int kCalibLds = 2 * kFinParts * kFinCols;

// lambda_j = 2 sum_s px[s][j], e_j = sum_s pw[s][j], score_j = lambda_j e_j,
// for the kFinCols columns of block blk. The order of the sums does not depend
// on the block's size: partial sum v (0 .. kFinParts - 1) takes the slices
// s = v (mod kFinParts) in order, and the partial sums are added in the order
// v = 0, 1, ...; thread t computes those of column t % kFinCols with
// v = t / kFinCols, t / kFinCols + blockDim.x / kFinCols, ...
__device__ __forceinline__ void fin_cols(const CalibLayer& L, int64_t blk, double* lds)
{
    double(&red)[2][kFinParts][kFinCols] = *reinterpret_cast<double(*)[2][kFinParts][kFinCols]>(lds);
    const int cl = threadIdx.x % kFinCols;
    const int64_t j = blk * kFinCols + cl;
    const int64_t jc = j < L.K ? j : L.K - 1;
    for (int v = threadIdx.x / kFinCols; v < kFinParts; v += blockDim.x / kFinCols) {
        double sx = 0.0, sw = 0.0;
#pragma unroll 2
        for (int64_t s = v; s < L.sx; s += kFinParts)
            sx += L.px[s * L.K + jc];
#pragma unroll 8
        for (int64_t s = v; s < L.sw; s += kFinParts)
            sw += L.pw[s * L.K + jc];
        red[0][v][cl] = sx;
        red[1][v][cl] = sw;
    }
    __syncthreads();
    if (threadIdx.x < kFinCols && j < L.K) {
        double lam = red[0][0][cl], e = red[1][0][cl];
        for (int v = 1; v < kFinParts; v++) {
            lam += red[0][v][cl];
            e += red[1][v][cl];
        }
        lam *= 2.0;
        L.lambda[j] = lam;
        L.score[j] = lam * e;
    }
}

// Final-sum and X blocks (every block at or after wb[count]); false: a W block
__device__ __forceinline__ bool fin_or_x_blocks(const CalibLaunch& c, int64_t b, double* lds)
{
    b -= c.wb[c.count];
    if (b < 0)
        return false;
    if (b < c.fb[c.count]) {
        const int l = layer_of(c.fb, c.count, b);
        fin_cols(c.L[l], b - c.fb[l], lds);
        return true;
    }
    b -= c.fb[c.count];
    const int l = layer_of(c.xb, c.count, b);
    const CalibLayer& L = c.L[l];
    b -= c.xb[l];
    colsum_tile(L.X, L.T, L.K, L.rows_x, L.px, SqElem{}, b % L.tiles, b / L.tiles,
                *reinterpret_cast<double(*)[kMaxWaves][kTileCols]>(lds));
    return true;
}

template <int WPL, int G, int D>
__global__ __launch_bounds__(1024) void k_calib_fused(const CalibLaunch c)
{
    __shared__ double lds[kCalibLds];
    __shared__ uint32_t mm[3][G][kMaxWaves];
    const int64_t b = blockIdx.x;
    if (fin_or_x_blocks(c, b, lds))
        return;
    const int l = layer_of(c.wb, c.count, b);
    const CalibLayer& L = c.L[l];
    const int64_t blk = b - c.wb[l];
    const int64_t r0 = blk * L.rows_w;
    fit_err_rows<WPL, G, D>(L.W, L.K, r0, min(L.N, r0 + L.rows_w), L.pw + blk * L.K, mm);
}

// two-pass form, first launch: row fits (one wave per row), final sums, X tiles
__global__ __launch_bounds__(256) void k_calib_fit(const CalibLaunch c)
{
    __shared__ double lds[kCalibLds];
    const int64_t b = blockIdx.x;
    if (fin_or_x_blocks(c, b, lds))
        return;
    const int l = layer_of(c.wb, c.count, b);
    const CalibLayer& L = c.L[l];
    rowfit_rows(L.W, L.N, L.K, L.s16, L.z, b - c.wb[l]);
}

// two-pass form, second launch: column tiles of the RTN errors
__global__ __launch_bounds__(256) void k_calib_err(const CalibLaunch c)
{
    __shared__ double red[kMaxWaves][kTileCols];
    int64_t b = blockIdx.x;
    const int l = layer_of(c.wb, c.count, b);
    const CalibLayer& L = c.L[l];
    b -= c.wb[l];
    colsum_tile(L.W, L.N, L.K, L.rows_w, L.pw, ErrElem{L.s16, L.z}, b % L.tiles, b / L.tiles, red);
}

// the final sums alone (after the last group of linears)
__global__ __launch_bounds__(1024) void k_calib_fin(const CalibLaunch c)
{
    __shared__ double lds[kCalibLds];
    const int64_t b = blockIdx.x;
    const int l = layer_of(c.fb, c.count, b);
    fin_cols(c.L[l], b - c.fb[l], lds);
}

// Rows per fused W block: one [K] fp64 partial row per block costs 4 / rows of
// W's bytes (12.5 % at 32); rows wider than kWpl2Words words take kFusedRowsWide
// (more, shorter blocks: such a block streams as many bytes as several narrow
// ones).
constexpr int64_t kFusedRows = 32;
constexpr int64_t kFusedRowsWide = 32;
// fused form: 2 words per lane up to kWpl2Words words per row (K = 8 x), 3 up to
// kWpl3Words, 4 above
constexpr int64_t kWpl2Words = 1024;
constexpr int64_t kWpl3Words = 1536;
// rows of X per tile block
constexpr int64_t kTileRows = 512;

// Row slices of a tile-form sum over R rows: kTileRows rows per block at most
int64_t choose_slices(int64_t R)
{
    int64_t s = (R + kTileRows - 1) / kTileRows;
    if (s > 65535)
        s = 65535;
    return s < 1 ? 1 : s;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

CalibPlan calib_plan(int64_t N, int64_t K, int64_t T)
{
    CalibPlan p;
    const int64_t nw = K / 8;
    if (nw <= kWpl2Words) {
        p.wpl = 2;
        p.nwaves = (int32_t)((nw + 127) / 128);
    } else if (nw <= kWpl3Words) {
        p.wpl = 3;
        p.nwaves = (int32_t)((nw + 191) / 192);
    } else if (nw <= 4096) {  // K <= 32768
        p.wpl = 4;
        p.nwaves = (int32_t)((nw + 255) / 256);
    } else {  // two-pass form
        p.wpl = 0;
        p.nwaves = 4;
    }
    p.sx = choose_slices(T);
    p.rows_x = (T + p.sx - 1) / p.sx;
    if (p.wpl) {
        p.rows_w = nw <= kWpl2Words ? kFusedRows : kFusedRowsWide;
        p.sw = (N + p.rows_w - 1) / p.rows_w;
    } else {
        p.sw = choose_slices(N);
        p.rows_w = (N + p.sw - 1) / p.sw;
    }
    size_t o = 0;
    p.off_px = o;
    o = align256(o + (size_t)p.sx * K * sizeof(double));
    p.off_pw = o;
    o = align256(o + (size_t)p.sw * K * sizeof(double));
    p.off_s16 = o;
    if (!p.wpl)
        o = align256(o + (size_t)N * sizeof(uint16_t));
    p.off_z = o;
    if (!p.wpl)
        o = align256(o + (size_t)N);
    p.total = o;
    return p;
}

hipError_t calib_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* dev_ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!dev_ptr[dev]) {  // first call on this device, with it current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        dev_ptr[dev] = p;
    }
    *ptr = dev_ptr[dev];
    return hipSuccess;
}

hipError_t launch_calibrate_batched(const CalibItem* items, int count, void* const* ws, const CalibPlan* plans,
                                   hipStream_t s)
{
    auto layer = [&](int l) {
        CalibLayer L;
        const CalibItem& it = items[l];
        const CalibPlan& p = plans[l];
        char* base = static_cast<char*>(ws[l]);
        L.W = it.W;
        L.X = it.X;
        L.px = reinterpret_cast<double*>(base + p.off_px);
        L.pw = reinterpret_cast<double*>(base + p.off_pw);
        L.s16 = reinterpret_cast<uint16_t*>(base + p.off_s16);
        L.z = reinterpret_cast<uint8_t*>(base + p.off_z);
        L.lambda = it.lambda;
        L.score = it.score;
        L.N = it.N;
        L.K = it.K;
        L.T = it.T;
        L.rows_x = p.rows_x;
        L.rows_w = p.rows_w;
        L.sx = p.sx;
        L.sw = p.sw;
        L.tiles = (it.K + kTileCols - 1) / kTileCols;
        return L;
    };
    // w_blocks / x_blocks: the W and X blocks of each linear of `ids` in one
    // launch; fin: linears whose final sums the launch also computes
    auto run = [&](const std::vector<int>& ids, const std::vector<int>& fin, auto kernel, int threads,
                   auto w_blocks, auto x_blocks) {
        CalibLaunch c{};
        const int n = (int)ids.size(), n2 = n + (int)fin.size();
        c.count = n2;
        c.wb[0] = c.fb[0] = c.xb[0] = 0;
        for (int i = 0; i < n2; i++) {
            const bool main = i < n;
            c.L[i] = layer(main ? ids[i] : fin[i - n]);
            c.wb[i + 1] = c.wb[i] + (int32_t)(main ? w_blocks(c.L[i]) : 0);
            c.fb[i + 1] = c.fb[i] + (int32_t)(main ? 0 : (c.L[i].K + kFinCols - 1) / kFinCols);
            c.xb[i + 1] = c.xb[i] + (int32_t)(main ? x_blocks(c.L[i]) : 0);
        }
        const int64_t nb = (int64_t)c.wb[n2] + c.fb[n2] + c.xb[n2];
        if (nb > 0)
            hipLaunchKernelGGL(kernel, dim3((unsigned)nb), dim3(threads), 0, s, c);
    };
    auto none = [](const CalibLayer&) { return (int64_t)0; };
    auto xtiles = [](const CalibLayer& L) { return L.tiles * L.sx; };
    auto fused = [](const CalibLayer& L) { return L.sw; };
    // linears of one block shape share a launch, kCalibChunk at a time; each
    // launch also finishes the previous chunk
    std::vector<int> pending;
    std::vector<char> done((size_t)count, 0);
    for (int l0 = 0; l0 < count; l0++) {
        if (done[l0])
            continue;
        std::vector<int> ids;
        for (int l = l0; l < count; l++)
            if (!done[l] && plans[l].wpl == plans[l0].wpl && plans[l].nwaves == plans[l0].nwaves) {
                ids.push_back(l);
                done[l] = 1;
            }
        const int wpl = plans[l0].wpl, threads = 64 * plans[l0].nwaves;
        for (size_t i = 0; i < ids.size(); i += kCalibChunk) {
            const std::vector<int> chunk(ids.begin() + i, ids.begin() + std::min(ids.size(), i + kCalibChunk));
            if (wpl == 2) {
                run(chunk, pending, k_calib_fused<2, 2, 1>, threads, fused, xtiles);
            } else if (wpl == 3) {
                run(chunk, pending, k_calib_fused<3, 2, 1>, threads, fused, xtiles);
            } else if (wpl == 4) {
                run(chunk, pending, k_calib_fused<4, 1, 1>, threads, fused, xtiles);
            } else {
                run(chunk, pending, k_calib_fit, 256, [](const CalibLayer& L) { return (L.N + 3) / 4; }, xtiles);
                run(chunk, {}, k_calib_err, 256, [](const CalibLayer& L) { return L.tiles * L.sw; }, none);
            }
            pending = chunk;
        }
    }
    run({}, pending, k_calib_fin, 1024, none, none);
    return hipGetLastError();
}

hipError_t launch_calibrate(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            double* lambda, double* score, void* ws, const CalibPlan& p,
                            hipStream_t s)
{
    CalibItem it{W, N, K, X, T, lambda, score};
    return launch_calibrate_batched(&it, 1, &ws, &p, s);
}

}  // namespace owq
