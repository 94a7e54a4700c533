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
// packed matrix, whose codes lie along K. One launch (k_bwd_part) covers two
// kinds of block:
//  * dw blocks (first token chunk only): dw_weak, below;
//  * dx blocks: 4 waves over one tile of 64 groups (2048 columns) and one
//    slice of rows; lane l decodes group l of the tile (the R7 slot layout gives
//    natural column pairs) and adds s_i dy[m][i] (q_ij - z_i) into 32 fp32
//    accumulators per token, one mixed-precision FMA per weight and token (the
//    fp16 (q - z) is exact). A wave loads 8 rows (4 at 3-4 tokens) before
//    it decodes any, so that many rows of codes are in flight; the 4 waves' sums are added in LDS in
//    wave order and the block writes one partial per slice. The weak columns
//    of the tile then add dy w_weak over the same rows (staged in LDS, rows in
//    order) to their column's partial.
// k_bwd_dx_finalize adds the slices' partials in a fixed order (8 phases of
// interleaved slices, then the phases in order) and rounds to fp16: results
// are bitwise deterministic. Token chunks of up to 4.
//
// dw_weak: a thread per row and 32 weak columns, x at the weak columns staged
// in LDS 64 tokens at a time, fp32 FMAs in token order.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kBwdMaxMT = 4;      // tokens per dx pass
constexpr int kTileGroups = 64;   // groups per column tile (one per lane)
constexpr int kWeakTile = 32;     // weak columns per block in the weak kernels
// rows per slice at least: every slice writes (and the finalize reads) 4 MT K
// bytes of partial sums. 64 against 32 rows: 57.5 -> 49.6 us for the 7 LLaMA-7B
// linears at M = 1, 115 -> 92 us at M = 4 (128: 48.0 and 97 us); loading a
// step's rows while the previous step is decoded did not help (56 us at M = 1)
constexpr int kBwdMinRows = 64;
// rows a wave loads before decoding: 8 at up to 2 tokens, else 4 (registers)
template <int MT>
constexpr int rows_in_flight() { return MT <= 2 ? 8 : 4; }

struct BwdArgs {
    const uint32_t* q;
    const uint16_t* scales;
    const uint8_t* zeros;
    const uint16_t* ww;
    const int32_t* idx;
    const uint16_t* dy;  // this chunk's tokens, [MT][N]
    const uint16_t* x;   // all tokens, [M][K] (dw blocks)
    float* P;            // partials [slices][MT][K]
    float* dw;           // [N][k]
    uint16_t* dx;        // this chunk's tokens, [MT][K]
    float* PW;           // matrix-core form: weak-column partials [slices][16][k]
    float* F;            // matrix-core form: fp32 column sums [16][K]
    int N, K, k, M, rows_per_slice, slices, tiles, dw_blocks, dx_blocks;
    int mt;              // tokens of this chunk (matrix-core form)
    int weak_blocks;     // matrix-core form: weak-partial blocks (slices x 16-column groups)
};

// The layers of one launch. Blocks: the dw blocks of every layer (layer l from
// dw0[l]), then the dx blocks of every layer (layer l from dx0[l], dx0[0] =
// dw0[count]); the finalize launch: layer l from f0[l].
struct BwdBatch {
    BwdArgs L[kBwdMaxLayers];
    int32_t dw0[kBwdMaxLayers + 1], dx0[kBwdMaxLayers + 1], f0[kBwdMaxLayers + 1];
    int32_t count;
};

// the layer whose block range [t[l], t[l + 1]) holds b (layers with no blocks
// are skipped: the last l with t[l] <= b)
__device__ __forceinline__ int layer_of(const int32_t* t, int count, int b)
{
    int li = 0;
    for (int l = 1; l < count; l++)
        if (b >= t[l])
            li = l;
    return li;
}

// dense block: partial sums of one token chunk over one row slice
template <int MT>
__device__ __forceinline__ void bwd_dense(const BwdArgs& a, int tile, int s, float* red)
{
    const int G = a.K >> 5;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = tile * kTileGroups + lane;
    const int gc = min(g, G - 1);  // lanes past the row's groups load a valid group and store nothing
    const int r0 = s * a.rows_per_slice, r1 = min(a.N, r0 + a.rows_per_slice);
    const Magic mg = make_magic();
    constexpr int kRowsInFlight = rows_in_flight<MT>();

    // The tile's weak columns are [c_lo, c_hi), c_lo = #{c : idx_c < j_lo}. With
    // at most 256 weak columns and a slice of at most 4096 weak weights, idx, the
    // slice's weak block (contiguous in w_weak) and its dy are loaded now, beside
    // the codes, by loads that are all unconditional (clamped indices; the
    // branch is block-uniform): the weak step after the dense sums then waits on
    // no load, and nothing here is waited for before the codes are requested.
    const int j_lo = tile * kTileGroups * 32, j_hi = min(a.K, j_lo + kTileGroups * 32);
    const int nrs = r1 - r0;
    const bool pre = a.k > 0 && a.k <= 256 && nrs * a.k <= 4096 && MT * nrs <= 256;
    // 32-bit registers: 16-bit values would be packed in pairs right after
    // loading, which waits for the loads
    uint32_t wv[16], dyh = 0;
    int idx_t = 0;
    if (pre) {
        const int t = threadIdx.x;
        idx_t = a.idx[min(t, a.k - 1)];
        const uint16_t* __restrict__ wsl = a.ww + (int64_t)r0 * a.k;
        const int last = nrs * a.k - 1;
#pragma unroll
        for (int u = 0; u < 16; u++)
            wv[u] = wsl[min(t + 256 * u, last)];
        const int m = min(t / nrs, MT - 1), r = t % nrs;
        dyh = a.dy[(int64_t)m * a.N + r0 + r];
    }

    float acc[MT][32];
#pragma unroll
    for (int m = 0; m < MT; m++)
#pragma unroll
        for (int c = 0; c < 32; c++)
            acc[m][c] = 0.0f;

    // wave w takes rows r0 + w + 4 t; kRowsInFlight of them per step, rows past
    // the slice load its last row and take a zero coefficient (adds exact zeros)
    struct Rows {
        uint32_t w[kRowsInFlight][3];
        uint16_t sh[kRowsInFlight], dh[kRowsInFlight][MT];
        uint32_t z[kRowsInFlight];
    };
    // every load of a step unconditional (rows clamped to the slice): a load
    // under a branch would be waited for at the branch's end, before the next
    // row's loads are issued
    auto load_rows = [&](int rb, Rows& R) {
#pragma unroll
        for (int u = 0; u < kRowsInFlight; u++) {
            const int rr = rb + 4 * u;
            const int r = rr < r1 ? rr : r1 - 1;
            const uint32_t* src = a.q + ((int64_t)r * G + gc) * 3;
            R.w[u][0] = src[0];
            R.w[u][1] = src[1];
            R.w[u][2] = src[2];
            R.sh[u] = a.scales[r];
            R.z[u] = a.zeros[r];
#pragma unroll
            for (int m = 0; m < MT; m++)
                R.dh[u][m] = a.dy[(int64_t)m * a.N + r];
        }
    };
    for (int rb = r0 + wave; rb < r1; rb += 4 * kRowsInFlight) {
        Rows R;
        load_rows(rb, R);
        auto& w = R.w;
        auto& sh = R.sh;
        auto& dh = R.dh;
        auto& z = R.z;
#pragma unroll
        for (int u = 0; u < kRowsInFlight; u++) {
            const bool live = rb + 4 * u < r1;
            const float sc = h2f(sh[u]);
            float coef[MT];
#pragma unroll
            for (int m = 0; m < MT; m++)
                coef[m] = live ? sc * h2f(dh[u][m]) : 0.0f;
            uint32_t p[16];
            decode_group(w[u][0], w[u][1], w[u][2], mg, make_zero_sub(z[u]), p);
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
    }
    // the 4 waves' sums, added in wave order; red is [3][32][64] floats
#pragma unroll
    for (int m = 0; m < MT; m++) {
        if (wave > 0)
#pragma unroll
            for (int c = 0; c < 32; c++)
                red[((wave - 1) * 32 + c) * 64 + lane] = acc[m][c];
        __syncthreads();
        if (wave == 0 && g < G) {
            float* dst = a.P + ((int64_t)s * MT + m) * a.K + (int64_t)g * 32;
#pragma unroll
            for (int c = 0; c < 32; c += 4) {
                float t[4];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    float v = acc[m][c + e];
                    v += red[(0 * 32 + c + e) * 64 + lane];
                    v += red[(1 * 32 + c + e) * 64 + lane];
                    v += red[(2 * 32 + c + e) * 64 + lane];
                    t[e] = v;
                }
                *reinterpret_cast<float4*>(dst + c) = make_float4(t[0], t[1], t[2], t[3]);
            }
        }
        __syncthreads();
    }
    if (a.k == 0)
        return;
    // the tile's weak columns [c_lo, c_hi): partial += sum over the slice's rows
    // (in order) of dy[m][i] w_weak[i][c]
    int n_lo = 0, n_hi = 0;
    if (pre) {
        // the prefetched values are first used here: this keeps the compiler
        // from moving their conversions (and so the wait) up to the loads
#pragma unroll
        for (int u = 0; u < 16; u++)
            asm volatile("" : "+v"(wv[u]));
        asm volatile("" : "+v"(dyh), "+v"(idx_t));
        const bool on = (int)threadIdx.x < a.k;
        n_lo = on && idx_t < j_lo;
        n_hi = on && idx_t < j_hi;
    } else {
        for (int c = threadIdx.x; c < a.k; c += 256) {
            const int v = a.idx[c];
            n_lo += v < j_lo;
            n_hi += v < j_hi;
        }
    }
    int* cnt = reinterpret_cast<int*>(red + 5120);  // 8 ints past the staging area
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        n_lo += __shfl_xor(n_lo, o, 64);
        n_hi += __shfl_xor(n_hi, o, 64);
    }
    if (lane == 0) {
        cnt[wave] = n_lo;
        cnt[4 + wave] = n_hi;
    }
    __syncthreads();
    const int c_lo = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    const int c_hi = cnt[4] + cnt[5] + cnt[6] + cnt[7];
    const int tid = threadIdx.x;
    if (pre) {
        // red[0, nrs k): the slice's weak weights (row-major), red[4096 + m nrs + r]:
        // dy, ids[c]: idx[c]; column c_lo + t sums its rows in order and adds the
        // total to the partial this block stored (the only add to that address)
        int* ids = reinterpret_cast<int*>(red + 5376);
        const int tot = nrs * a.k;
#pragma unroll
        for (int u = 0; u < 16; u++) {
            const int e = tid + 256 * u;
            if (e < tot)
                red[e] = h2f((uint16_t)wv[u]);
        }
        if (tid < MT * nrs)
            red[4096 + tid] = h2f((uint16_t)dyh);
        if (tid < a.k)
            ids[tid] = idx_t;
        __syncthreads();
        const int c = c_lo + tid;
        if (c < c_hi) {
            float wacc[MT];
#pragma unroll
            for (int m = 0; m < MT; m++)
                wacc[m] = 0.0f;
            for (int r = 0; r < nrs; r++) {
                const float w = red[r * a.k + c];
#pragma unroll
                for (int m = 0; m < MT; m++)
                    wacc[m] = __builtin_fmaf(red[4096 + m * nrs + r], w, wacc[m]);
            }
            const int j = ids[c];
#pragma unroll
            for (int m = 0; m < MT; m++)
                (void)unsafeAtomicAdd(a.P + ((int64_t)s * MT + m) * a.K + j, wacc[m]);
        }
        return;
    }
    // general form: 64 columns x 64 rows staged at a time
    for (int cb = c_lo; cb < c_hi; cb += 64) {
        const int nc = min(64, c_hi - cb);
        float wacc[MT];
#pragma unroll
        for (int m = 0; m < MT; m++)
            wacc[m] = 0.0f;
        for (int rb = r0; rb < r1; rb += 64) {
            const int nr = min(64, r1 - rb);
            // nr x nc weights, element e at (e / nc, e % nc): every load issued
            // before the first LDS store
            const int tot = nr * nc;
            uint16_t v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int e = tid + 256 * u;
                const int r = e / nc, c = e - r * nc;
                v[u] = e < tot ? a.ww[(int64_t)(rb + r) * a.k + cb + c] : (uint16_t)0;
            }
            const float dv = tid < MT * 64 && (tid & 63) < nr ? h2f(a.dy[(int64_t)(tid >> 6) * a.N + rb + (tid & 63)])
                                                               : 0.0f;
#pragma unroll
            for (int u = 0; u < 16; u++) {
                const int e = tid + 256 * u;
                const int r = e / nc, c = e - r * nc;
                if (e < tot)
                    red[r * 64 + c] = h2f(v[u]);
            }
            if (tid < MT * 64)  // dy of the staged rows after the block: red[4096 + m * 64 + r]
                red[4096 + tid] = dv;
            __syncthreads();
            if (tid < nc)
                for (int r = 0; r < nr; r++) {
                    const float w = red[r * 64 + tid];
#pragma unroll
                    for (int m = 0; m < MT; m++)
                        wacc[m] = __builtin_fmaf(red[4096 + m * 64 + r], w, wacc[m]);
                }
            __syncthreads();
        }
        if (tid < nc) {
            // the partial at a weak column was stored above by this block; this
            // is the only add to it
            const int j = a.idx[cb + tid];
#pragma unroll
            for (int m = 0; m < MT; m++)
                (void)unsafeAtomicAdd(a.P + ((int64_t)s * MT + m) * a.K + j, wacc[m]);
        }
    }
}

// dw block: dw[i][c] = sum_m dy[m][i] x[m][idx_c], a thread per row, 32 weak
// columns; a.dy here points at token 0. x at the block's weak columns is staged
// in LDS 64 tokens at a time. The first loads (the column indices, dy of the
// first tokens) are issued together and unconditionally (clamped), and every x
// load of a stage before the first LDS store, so the chain is indices -> x.
__device__ __forceinline__ void bwd_dw(const BwdArgs& a, int bi, float* xs)
{
    // 256 working threads; in a larger block the others pass the barriers only
    const int tid = threadIdx.x & 255;
    const bool on = threadIdx.x < 256;
    constexpr int MC = 64, MD = 16;  // tokens per stage; dy values loaded up front
    int* cols = reinterpret_cast<int*>(xs + MC * kWeakTile);
    const int rt = (a.N + 255) / 256;
    const int i = (bi % rt) * 256 + tid;
    const int c0 = (bi / rt) * kWeakTile;
    const int nc = min(kWeakTile, a.k - c0);
    const int ic = min(i, a.N - 1);
    const int jl = a.idx[c0 + min(tid & (kWeakTile - 1), nc - 1)];
    float* dys = xs + MC * kWeakTile + 64;  // [MD][256]: dy of the first tokens
    uint32_t d0[MD];
#pragma unroll
    for (int mm = 0; mm < MD; mm++)
        d0[mm] = a.dy[(int64_t)min(mm, a.M - 1) * a.N + ic];
    if (on && tid < kWeakTile)
        cols[tid] = (jl >= 0 && jl < a.K) ? jl : 0;
    if (on)
#pragma unroll
        for (int mm = 0; mm < MD; mm++)
            dys[mm * 256 + tid] = h2f((uint16_t)d0[mm]);
    float acc[kWeakTile];
#pragma unroll
    for (int c = 0; c < kWeakTile; c++)
        acc[c] = 0.0f;
    for (int m0 = 0; m0 < a.M; m0 += MC) {
        const int mn = min(MC, a.M - m0);
        __syncthreads();  // cols written / the previous tokens' x no longer read
        uint32_t v[MC * kWeakTile / 256];
#pragma unroll
        for (int u = 0; u < MC * kWeakTile / 256; u++) {
            const int e = tid + 256 * u;
            const int mm = e / kWeakTile, cc = e % kWeakTile;
            v[u] = a.x[(int64_t)(m0 + min(mm, mn - 1)) * a.K + cols[cc]];
        }
        if (on)
#pragma unroll
            for (int u = 0; u < MC * kWeakTile / 256; u++) {
                const int e = tid + 256 * u;
                const int mm = e / kWeakTile, cc = e % kWeakTile;
                xs[e] = (mm < mn && cc < nc) ? h2f((uint16_t)v[u]) : 0.0f;
            }
        __syncthreads();
        for (int mm = 0; mm < mn; mm++) {
            const int m = m0 + mm;
            const float d = m < MD ? dys[m * 256 + tid] : h2f(a.dy[(int64_t)m * a.N + ic]);
#pragma unroll
            for (int c = 0; c < kWeakTile; c++)
                acc[c] = __builtin_fmaf(d, xs[mm * kWeakTile + c], acc[c]);
        }
    }
    if (on && i < a.N)
        for (int c = 0; c < nc; c++)
            a.dw[(int64_t)i * a.k + c0 + c] = acc[c];
}

// blocks [0, dw0[count]): dw (first, so that their short dependent chains run
// beside the dx blocks rather than after them), then the dx blocks of each layer
// (slice-major within a tile column)
template <int MT>
__global__ __launch_bounds__(256) void k_bwd_part(const BwdBatch bt)
{
    __shared__ float red[3 * 32 * 64 + 128];  // 24.5 KiB, shared by the two roles
    const int b = blockIdx.x;
    if (b < bt.dw0[bt.count]) {
        const int li = layer_of(bt.dw0, bt.count, b);
        bwd_dw(bt.L[li], b - bt.dw0[li], red);
        return;
    }
    const int li = layer_of(bt.dx0, bt.count, b);
    const BwdArgs& a = bt.L[li];
    const int bb = b - bt.dx0[li];
    bwd_dense<MT>(a, bb % a.tiles, bb / a.tiles, red);
}

// dx[m][j] = fp16(sum over the slices' partials). 32 columns x 8 phases per
// block: phase f sums slices f, f+8, ... in order (8 loads in flight); the
// phases are then added in order.
template <int MT>
__global__ __launch_bounds__(256) void k_bwd_dx_finalize(const BwdBatch bt)
{
    __shared__ float red[8][32];
    const int li = layer_of(bt.f0, bt.count, blockIdx.x);
    const BwdArgs& a = bt.L[li];
    const int K = a.K, slices = a.slices;
    const int col = threadIdx.x & 31, ph = threadIdx.x >> 5;
    const int64_t e = (int64_t)(blockIdx.x - bt.f0[li]) * 32 + col;  // m * K + j within the chunk
    const int64_t n = (int64_t)MT * K;
    const bool ok = e < n;
    const float* __restrict__ p = a.P + (ok ? e : 0);
    float t = 0.0f;
    if (ok) {
        int s = ph;
        for (; s + 56 < slices; s += 64) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; u++)
                v[u] = p[(int64_t)(s + 8 * u) * n];
#pragma unroll
            for (int u = 0; u < 8; u++)
                t += v[u];
        }
        for (; s < slices; s += 8)
            t += p[(int64_t)s * n];
    }
    red[ph][col] = t;
    __syncthreads();
    if (ph != 0 || !ok)
        return;
    t = red[0][col];
#pragma unroll
    for (int f = 1; f < 8; f++)
        t += red[f][col];
    a.dx[e] = f2h(t);
}

// ---------------------------------------------------------------------------
// Matrix-core form of dx for more than 4 tokens, 16 per pass. The contraction
// runs over the rows i, while a lane's decoded group holds 32 columns of one
// row, so the decoded codes go through LDS: a block (4 waves) owns 256 columns
// (8 groups) and one slice of rows; per step of 32 rows, thread t decodes group
// t % 8 of row t / 8 into the LDS tile (exact (q - z) fp16, natural column
// order), and the step's dy (fp16, 16 tokens) and steps s_i go to LDS beside it.
// Each wave then multiplies its 64 columns with v_mfma_f32_16x16x32_f16:
// A[m][r] = dy[m][i] (exact), B[r][j] = s_i (q_ij - z_i) as the exact sum of two
// fp16 values B_hi = fp16(s (q - z)) (v_pk_mul_f16) and B_lo = s (q - z) - B_hi
// (v_pk_fma_f16, exact: s (q - z) is a multiple of s's last bit with at most 14
// significant bits, so the remainder has at most 3 and lies on fp16's grid, also
// where it is subnormal), two MFMAs per 32 rows. Every product dy B_hi, dy B_lo
// is exact in fp32 and only the sums round, as in the vector form. The k index
// of the MFMA (8 (l / 16) + e for lane l, operand element e) takes the step's
// row 4 e + l / 16, so the four rows of one B read are consecutive (distinct
// banks with the padded tile rows); the dy tile is stored in that order.
// B_hi overflows fp16 only if s (q - z) > 65504, i.e. s > 9352: a block whose
// row slice holds such a row multiplies in fp32 instead (v_mfma_f32_16x16x4_f32
// with A = s_i dy[m][i], exact in fp32, B = q - z); the two forms are separate
// loops, so neither carries the other's accumulator copies. The tile is
// double-buffered (one barrier per step) and
// the next step's loads are issued before this step's products. The block
// stores its partial sums P[slice][m][j].
constexpr int kMmaCols = 256;  // columns per block
constexpr int kMmaRows = 32;   // rows per step
constexpr int kMmaRowBytes = kMmaCols * 2 + 64;  // LDS row of the decoded tile (padded: 144 dwords, the
                                                 // four rows of a B read on distinct banks)
constexpr uint16_t kMmaMaxStep = 0x7091;  // fp16 9352: 7 s <= 65504

typedef float f32x4 __attribute__((ext_vector_type(4)));

// position of step row r in the dy and step tiles: row 4 e + c at 8 c + e
__device__ __forceinline__ int mma_kpos(int r) { return 8 * (r & 3) + (r >> 2); }

__device__ __forceinline__ half8_t mma_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    return __builtin_bit_cast(half8_t, make_uint4(a, b, c, d));
}

__device__ __forceinline__ void bwd_mma_dense(const BwdArgs& a, int tile, int s, char* lds)
{
    char* const tw = lds;  // [2][32][kMmaRowBytes]
    // [2][16][32] dy (token-major, rows at mma_kpos), then [2][32] steps
    uint16_t* const tdy = reinterpret_cast<uint16_t*>(lds + 2 * kMmaRows * kMmaRowBytes);
    uint16_t* const tsv = tdy + 2 * 16 * kMmaRows;
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int G = a.K >> 5;
    const int lrow = t >> 3, lg = t & 7;
    const int g = min(tile * 8 + lg, G - 1);  // groups past K decode a valid group; their columns are not stored
    const int r0 = s * a.rows_per_slice, r1 = min(a.N, r0 + a.rows_per_slice);
    const int nsteps = (r1 - r0 + kMmaRows - 1) / kMmaRows;
    const Magic mg = make_magic();
    // loads of step st: the row's group and, for the entries e = t and t + 256
    // of the 32 x 16 dy tile (row e / 16, token e % 16), s and dy
    uint32_t w0, w1, w2, zb;
    uint32_t sh[2], dh[2];
    auto issue = [&](int st) {
        const int rr = r0 + st * kMmaRows + lrow;
        const int r = min(rr, r1 - 1);
        const uint32_t* src = a.q + ((int64_t)r * G + g) * 3;
        w0 = src[0];
        w1 = src[1];
        w2 = src[2];
        zb = a.zeros[r];
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int e = t + 256 * h;
            const int cr = min(r0 + st * kMmaRows + (e >> 4), r1 - 1);
            const int m = min(e & 15, a.mt - 1);
            sh[h] = a.scales[cr];
            dh[h] = a.dy[(int64_t)m * a.N + cr];
        }
    };
    // step st's tiles into buffer st & 1 (rows past the slice and tokens past
    // the chunk get dy = 0)
    auto stage = [&](int st) {
        const int buf = st & 1;
        uint32_t p[16];
        decode_group(w0, w1, w2, mg, make_zero_sub(zb), p);
        // 16-byte chunk q of group lg at slot q ^ (lg >> 2): the lanes lg and lg + 4
        // of a 16-lane write pass then start on different banks
        uint4* dst = reinterpret_cast<uint4*>(tw + (buf * kMmaRows + lrow) * kMmaRowBytes + lg * 64);
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
            dst[q4 ^ (lg >> 2)] = make_uint4(p[4 * q4], p[4 * q4 + 1], p[4 * q4 + 2], p[4 * q4 + 3]);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const int e = t + 256 * h;
            const int r = e >> 4, m = e & 15;
            const bool row_live = r0 + st * kMmaRows + r < r1;
            tdy[(buf * 16 + m) * kMmaRows + mma_kpos(r)] = row_live && m < a.mt ? (uint16_t)dh[h] : (uint16_t)0;
            if (m == 0)
                tsv[buf * kMmaRows + mma_kpos(r)] = (uint16_t)sh[h];
        }
    };
    const int kg = lane >> 4, l16 = lane & 15;
    // the dword of column pair (c, c + 1), c = 64 w + 32 pb + 2 (l % 16), in a tile row
    int boff[2];
#pragma unroll
    for (int pb = 0; pb < 2; pb++) {
        const int col = 64 * wave + 32 * pb + 2 * l16;
        const int cg = col >> 5, cq = (col >> 3) & 3;  // group, 16-byte chunk
        boff[pb] = cg * 64 + ((cq ^ (cg >> 2)) << 4) + (col & 7) * 2;
    }
    // a step above kMmaMaxStep anywhere in the slice: the block multiplies in
    // fp32 (flag word after the step tiles, cleared before the first barrier)
    int* const tbig = reinterpret_cast<int*>(tsv + 2 * kMmaRows);
    if (t == 0)
        *tbig = 0;
    issue(0);
    bool big = false;
    for (int r = r0 + t; r < r1; r += 256)
        big = big || a.scales[r] > kMmaMaxStep;
    __syncthreads();
    if (big)
        *tbig = 1;
    stage(0);
    if (nsteps > 1)
        issue(1);
    __syncthreads();
    big = *tbig != 0;  // block-uniform
    // the step loop with the products of one form; accumulator 2 pb + h holds
    // the even (h = 0) or odd columns of pair block pb
    auto run = [&](auto fp16_form) {
        constexpr bool kF16 = decltype(fp16_form)::value;
        // acc: the fp32 form's sums or the fp16 form's B_hi products; accl: the
        // B_lo products (apart, so that no MFMA waits on the one before it)
        f32x4 acc[4], accl[4];
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            acc[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            accl[cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        for (int st = 0; st < nsteps; st++) {
            const int buf = st & 1;
            // this step's operands into registers and its products; then the
            // next step's tiles into the other buffer
            const char* trow = tw + buf * kMmaRows * kMmaRowBytes;
            if constexpr (kF16) {
                // A: dy of token l % 16 at rows 4 e + l / 16; steps of the same rows, in pairs
                const half8_t av = *reinterpret_cast<const half8_t*>(tdy + (buf * 16 + l16) * kMmaRows + 8 * kg);
                const uint4 sq = *reinterpret_cast<const uint4*>(tsv + buf * kMmaRows + 8 * kg);
                const uint32_t sp[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
                for (int pb = 0; pb < 2; pb++) {
                    uint32_t d[8];
#pragma unroll
                    for (int e = 0; e < 8; e++)
                        d[e] = *reinterpret_cast<const uint32_t*>(trow + (4 * e + kg) * kMmaRowBytes + boff[pb]);
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        // (q - z) of column 2 (l % 16) + h at rows 4 e + l / 16, e = 2 i, 2 i + 1
                        uint32_t bh[4], bl[4];
#pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const uint32_t qz =
                                __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], h ? 0x07060302u : 0x05040100u);
                            const half2_t sv = as_h2(sp[i]), qv = as_h2(qz);
                            const half2_t hi = sv * qv;
                            const half2_t lo = __builtin_elementwise_fma(sv, qv, -hi);
                            bh[i] = __builtin_bit_cast(uint32_t, hi);
                            bl[i] = __builtin_bit_cast(uint32_t, lo);
                        }
                        const int cb = 2 * pb + h;
                        acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, mma_h8(bh[0], bh[1], bh[2], bh[3]), acc[cb],
                                                                          0, 0, 0);
                        accl[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, mma_h8(bl[0], bl[1], bl[2], bl[3]),
                                                                           accl[cb], 0, 0, 0);
                    }
                }
            } else {
                // k-step ks takes rows 4 ks + l / 16; A = s dy (exact in fp32), B = q - z
#pragma unroll
                for (int ks = 0; ks < kMmaRows / 4; ks++) {
                    const int kr = 4 * ks + kg;
                    const float av = h2f(tsv[buf * kMmaRows + mma_kpos(kr)]) *
                                     h2f(tdy[(buf * 16 + l16) * kMmaRows + mma_kpos(kr)]);
#pragma unroll
                    for (int pb = 0; pb < 2; pb++) {
                        const half2_t hp =
                            as_h2(*reinterpret_cast<const uint32_t*>(trow + kr * kMmaRowBytes + boff[pb]));
                        acc[2 * pb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, (float)hp.x, acc[2 * pb], 0, 0, 0);
                        acc[2 * pb + 1] =
                            __builtin_amdgcn_mfma_f32_16x16x4f32(av, (float)hp.y, acc[2 * pb + 1], 0, 0, 0);
                    }
                }
            }
            if (st + 1 < nsteps) {
                stage(st + 1);
                if (st + 2 < nsteps)
                    issue(st + 2);
            }
            __syncthreads();
        }
        // D element r of lane l: token 4 (l / 16) + r; accumulator cb = 2 pb + h:
        // column 64 w + 32 pb + 2 (l % 16) + h
#pragma unroll
        for (int cb = 0; cb < 4; cb++) {
            const int j = tile * kMmaCols + 64 * wave + 32 * (cb >> 1) + 2 * (lane & 15) + (cb & 1);
            if (j < a.K)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    const int m = 4 * (lane >> 4) + r;
                    if (m < a.mt)
                        a.P[((int64_t)s * 16 + m) * a.K + j] = kF16 ? acc[cb][r] + accl[cb][r] : acc[cb][r];
                }
        }
    };
    if (big)
        run(std::false_type{});
    else
        run(std::true_type{});
}

// weak-column partials of one row slice: PW[slice][m][c] = sum over the slice's
// rows (in order) of dy[m][i] w_weak[i][c], 16 columns per block, thread (c, m),
// 64 rows staged in LDS at a time (every load of a stage issued before the
// first LDS store)
__device__ __forceinline__ void bwd_mma_weak(const BwdArgs& a, int cg, int s, char* lds)
{
    float* const dyl = reinterpret_cast<float*>(lds);  // [16][64]
    float* const wl = dyl + 16 * 64;                    // [64][16]
    // 256 working threads; in a larger block the others pass the barriers only
    const int t = threadIdx.x & 255;
    const bool on = threadIdx.x < 256;
    const int cl = t >> 4, m = t & 15;
    const int c0 = cg * 16;
    const int r0 = s * a.rows_per_slice, r1 = min(a.N, r0 + a.rows_per_slice);
    float acc = 0.0f;
    for (int rb = r0; rb < r1; rb += 64) {
        const int nr = min(64, r1 - rb);
        uint32_t dv[4], wv[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int e = t + 256 * u;  // dy: token e / 64, row e % 64; w: row e / 16, column e % 16
            const int dm = min(e >> 6, a.mt - 1), dr = min(e & 63, nr - 1);
            dv[u] = a.dy[(int64_t)dm * a.N + rb + dr];
            const int wr = min(e >> 4, nr - 1), wc = min(c0 + (e & 15), a.k - 1);
            wv[u] = a.ww[(int64_t)(rb + wr) * a.k + wc];
        }
        __syncthreads();  // the previous stage is no longer read
        if (on)
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int e = t + 256 * u;
                dyl[e] = (e >> 6) < a.mt && (e & 63) < nr ? h2f((uint16_t)dv[u]) : 0.0f;
                wl[e] = (e >> 4) < nr && c0 + (e & 15) < a.k ? h2f((uint16_t)wv[u]) : 0.0f;
            }
        __syncthreads();
        for (int r = 0; r < nr; r++)
            acc = __builtin_fmaf(dyl[m * 64 + r], wl[r * 16 + cl], acc);
    }
    if (on && c0 + cl < a.k && m < a.mt)
        a.PW[((int64_t)s * 16 + m) * a.k + c0 + cl] = acc;
}

// blocks: the dw_weak blocks of every layer (layer l from f0[l]; f0[count] =
// dw0[0]), the weak-partial blocks (layer l from dw0[l]), then the dense blocks
// (layer l from dx0[l])
__global__ __launch_bounds__(256) void k_bwd_mma(const BwdBatch bt)
{
    __shared__ __attribute__((aligned(16))) char lds[2 * kMmaRows * kMmaRowBytes + 2 * kMmaRows * 16 * 4];
    const int b = blockIdx.x;
    if (b < bt.f0[bt.count]) {
        const int li = layer_of(bt.f0, bt.count, b);
        bwd_dw(bt.L[li], b - bt.f0[li], reinterpret_cast<float*>(lds));
        return;
    }
    if (b < bt.dw0[bt.count]) {
        const int li = layer_of(bt.dw0, bt.count, b);
        const BwdArgs& a = bt.L[li];
        const int bb = b - bt.dw0[li];
        const int ngrp = (a.k + 15) / 16;
        bwd_mma_weak(a, bb % ngrp, bb / ngrp, lds);
        return;
    }
    const int li = layer_of(bt.dx0, bt.count, b);
    const BwdArgs& a = bt.L[li];
    const int bb = b - bt.dx0[li];
    bwd_mma_dense(a, bb % a.tiles, bb / a.tiles, lds);
}

// dx[m][j] = fp16(sum over the slices' partials, in slice order), and the fp32
// sum to F for the weak columns' correction; a thread per output, 8 partials
// loaded at a time
__global__ __launch_bounds__(256) void k_bwd_mma_finalize(const BwdBatch bt)
{
    const int li = layer_of(bt.f0, bt.count, blockIdx.x);
    const BwdArgs& a = bt.L[li];
    const int K = a.K, slices = a.slices;
    const int64_t e = (int64_t)(blockIdx.x - bt.f0[li]) * 256 + threadIdx.x;  // m * K + j, m < mt
    const int64_t n = (int64_t)a.mt * K, stride = (int64_t)16 * K;
    if (e >= n)
        return;
    const float* __restrict__ p = a.P + e;
    float t = 0.0f;
    int s = 0;
    for (; s + 8 <= slices; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            v[u] = p[(int64_t)(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; u++)
            t += v[u];
    }
    for (; s < slices; s++)
        t += p[(int64_t)s * stride];
    a.dx[e] = f2h(t);
    if (a.k > 0)
        a.F[e] = t;
}

// the weak columns: dx[m][idx_c] = fp16(F[m][idx_c] + sum over the slices of
// PW[s][m][c]) (the dense codes there are the zero point, but their partial is
// added as for any column); a thread per (c, m)
__global__ __launch_bounds__(256) void k_bwd_mma_weak_finalize(const BwdBatch bt)
{
    const int li = layer_of(bt.f0, bt.count, blockIdx.x);
    const BwdArgs& a = bt.L[li];
    const int64_t e = (int64_t)(blockIdx.x - bt.f0[li]) * 256 + threadIdx.x;  // c * 16 + m
    const int c = (int)(e >> 4), m = (int)(e & 15);
    if (c >= a.k || m >= a.mt)
        return;
    const int j = a.idx[c];
    const float* __restrict__ pw = a.PW + (int64_t)m * a.k + c;
    const int64_t stride = (int64_t)16 * a.k;
    float w = 0.0f;
    int s = 0;
    for (; s + 8 <= a.slices; s += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; u++)
            v[u] = pw[(int64_t)(s + u) * stride];
#pragma unroll
        for (int u = 0; u < 8; u++)
            w += v[u];
    }
    for (; s < a.slices; s++)
        w += pw[(int64_t)s * stride];
    a.dx[(int64_t)m * a.K + j] = f2h(a.F[(int64_t)m * a.K + j] + w);
}

// one 16-token chunk of every layer in bt on the matrix cores
hipError_t mma_chunk_launch(BwdBatch& bt, hipStream_t s)
{
    int nb = 0;
    for (int l = 0; l < bt.count; l++) {  // dw_weak blocks (first chunk only)
        bt.f0[l] = nb;
        nb += bt.L[l].dw_blocks;
    }
    bt.f0[bt.count] = nb;
    for (int l = 0; l < bt.count; l++) {
        bt.dw0[l] = nb;
        nb += bt.L[l].weak_blocks;
    }
    bt.dw0[bt.count] = nb;
    for (int l = 0; l < bt.count; l++) {
        bt.dx0[l] = nb;
        nb += bt.L[l].dx_blocks;
    }
    bt.dx0[bt.count] = nb;
    if (nb > 0)
        hipLaunchKernelGGL(k_bwd_mma, dim3((unsigned)nb), dim3(256), 0, s, bt);
    int nf = 0;
    for (int l = 0; l < bt.count; l++) {
        bt.f0[l] = nf;
        nf += bt.L[l].dx_blocks > 0 ? (int)((bt.L[l].mt * (int64_t)bt.L[l].K + 255) / 256) : 0;
    }
    bt.f0[bt.count] = nf;
    if (nf > 0)
        hipLaunchKernelGGL(k_bwd_mma_finalize, dim3((unsigned)nf), dim3(256), 0, s, bt);
    int nw = 0;
    for (int l = 0; l < bt.count; l++) {
        bt.f0[l] = nw;
        nw += bt.L[l].weak_blocks > 0 ? (int)((16 * (int64_t)bt.L[l].k + 255) / 256) : 0;
    }
    bt.f0[bt.count] = nw;
    if (nw > 0)
        hipLaunchKernelGGL(k_bwd_mma_weak_finalize, dim3((unsigned)nw), dim3(256), 0, s, bt);
    return hipGetLastError();
}

// one token chunk of every layer in bt (dy / dx already at the chunk): the part
// launch, then the finalize launch of the layers that want dx
template <int MT>
hipError_t chunk_launch(BwdBatch& bt, hipStream_t s)
{
    int nb = 0;
    for (int l = 0; l < bt.count; l++) {
        bt.dw0[l] = nb;
        nb += bt.L[l].dw_blocks;
    }
    bt.dw0[bt.count] = nb;
    for (int l = 0; l < bt.count; l++) {
        bt.dx0[l] = nb;
        nb += bt.L[l].dx_blocks;
    }
    bt.dx0[bt.count] = nb;
    int nf = 0;
    for (int l = 0; l < bt.count; l++) {
        bt.f0[l] = nf;
        nf += bt.L[l].dx_blocks > 0 ? (int)((MT * (int64_t)bt.L[l].K + 31) / 32) : 0;
    }
    bt.f0[bt.count] = nf;
    if (nb > 0)
        hipLaunchKernelGGL((k_bwd_part<MT>), dim3((unsigned)nb), dim3(256), 0, s, bt);
    if (nf > 0)
        hipLaunchKernelGGL((k_bwd_dx_finalize<MT>), dim3((unsigned)nf), dim3(256), 0, s, bt);
    return hipGetLastError();
}

}  // namespace

BwdPlan bwd_plan(int64_t N, int64_t K, int32_t k)
{
    BwdPlan p;
    // enough dense blocks to fill the GPU (512, two per CU) with slices of at
    // least kBwdMinRows rows, the partial sums (4 tokens, K columns, fp32 per
    // slice) within 64 MiB
    const int64_t tiles = (K / 32 + kTileGroups - 1) / kTileGroups;
    int64_t sl = (512 + tiles - 1) / tiles;
    const int64_t most = (N + kBwdMinRows - 1) / kBwdMinRows;
    const int64_t cap = ((int64_t)64 << 20) / (kBwdMaxMT * K * (int64_t)sizeof(float));
    if (sl > most)
        sl = most;
    if (sl > cap)
        sl = cap;
    p.slices = sl < 1 ? 1 : sl;
    p.rows_per_slice = (N + p.slices - 1) / p.slices;
    p.slices = (N + p.rows_per_slice - 1) / p.rows_per_slice;  // no empty slice
    auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
    p.off_p = 0;
    const size_t vec_total = al((size_t)p.slices * kBwdMaxMT * K * sizeof(float));
    // matrix-core form: slices of 512 rows (a multiple of the 32-row step)
    p.m_rows = 512;
    p.m_slices = (N + p.m_rows - 1) / p.m_rows;
    p.m_off_p = 0;
    p.m_off_pw = al((size_t)p.m_slices * 16 * K * sizeof(float));
    p.m_off_f = p.m_off_pw + al((size_t)p.m_slices * 16 * (k > 0 ? k : 1) * sizeof(float));
    const size_t mma_total = p.m_off_f + al((size_t)16 * K * sizeof(float));
    p.total = vec_total > mma_total ? vec_total : mma_total;
    return p;
}

// The matrix-core form for more than 4 tokens; OWQ_BACKWARD=vector (read at
// each call) keeps the vector form at every M.
bool mma_backward_enabled()
{
    const char* e = std::getenv("OWQ_BACKWARD");
    return !(e && std::strcmp(e, "vector") == 0);
}

hipError_t launch_linear_backward_batched(const LinearDesc* d, const uint16_t* const* dy, int count, int64_t M,
                                          uint16_t* const* dx, float* const* dw, void* const* ws,
                                          const BwdPlan* p, hipStream_t s)
{
    BwdBatch bt{};
    bt.count = count;
    bool any_dx = false;
    for (int l = 0; l < count; l++) {
        BwdArgs& a = bt.L[l];
        a.q = d[l].q;
        a.scales = d[l].s;
        a.zeros = d[l].z;
        a.ww = d[l].ww;
        a.idx = d[l].idx;
        a.dy = dy[l];
        a.x = d[l].x;
        a.P = (dx[l] && ws[l]) ? reinterpret_cast<float*>(static_cast<char*>(ws[l]) + p[l].off_p) : nullptr;
        a.dw = dw[l];
        a.dx = dx[l];
        a.N = (int)d[l].N;
        a.K = (int)d[l].K;
        a.k = d[l].k;
        a.M = (int)M;
        a.rows_per_slice = (int)p[l].rows_per_slice;
        a.slices = (int)p[l].slices;
        a.tiles = (int)((d[l].K / 32 + kTileGroups - 1) / kTileGroups);
        a.dw_blocks = (dw[l] && d[l].k > 0) ? (int)((d[l].N + 255) / 256) * ((d[l].k + kWeakTile - 1) / kWeakTile) : 0;
        a.dx_blocks = dx[l] ? a.slices * a.tiles : 0;
        any_dx = any_dx || dx[l];
    }
    if (!any_dx)  // dw only: the dw blocks alone (the token count does not matter)
        return chunk_launch<1>(bt, s);
    if (M > kBwdMaxMT && mma_backward_enabled()) {
        // dx: 16 tokens per pass on the matrix cores; dw_weak: blocks of the
        // first pass's launch (they read every token, from dy at token 0)
        hipError_t e = hipSuccess;
        for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += 16) {
            BwdBatch c = bt;
            for (int l = 0; l < count; l++) {
                BwdArgs& a = c.L[l];
                char* base = static_cast<char*>(ws[l]);
                a.dy = dy[l] + m0 * d[l].N;
                a.dx = dx[l] ? dx[l] + m0 * d[l].K : nullptr;
                a.mt = (int)(M - m0 < 16 ? M - m0 : 16);
                a.rows_per_slice = (int)p[l].m_rows;
                a.slices = (int)p[l].m_slices;
                a.tiles = (int)((d[l].K + kMmaCols - 1) / kMmaCols);
                a.P = dx[l] ? reinterpret_cast<float*>(base + p[l].m_off_p) : nullptr;
                a.PW = dx[l] ? reinterpret_cast<float*>(base + p[l].m_off_pw) : nullptr;
                a.F = dx[l] ? reinterpret_cast<float*>(base + p[l].m_off_f) : nullptr;
                a.dx_blocks = dx[l] ? a.slices * a.tiles : 0;
                a.weak_blocks = (dx[l] && d[l].k > 0) ? a.slices * ((d[l].k + 15) / 16) : 0;
                if (m0 > 0)
                    a.dw_blocks = 0;
            }
            e = mma_chunk_launch(c, s);
        }
        return e;
    }
    hipError_t e = hipSuccess;
    for (int64_t m0 = 0; m0 < M && e == hipSuccess; m0 += kBwdMaxMT) {
        const int mt = (int)(M - m0 < kBwdMaxMT ? M - m0 : kBwdMaxMT);
        BwdBatch c = bt;
        for (int l = 0; l < count; l++) {
            BwdArgs& a = c.L[l];
            a.dy = dy[l] + m0 * d[l].N;  // the dw blocks read every token from dy at token 0
            a.dx = dx[l] ? dx[l] + m0 * d[l].K : nullptr;
            if (m0 > 0)
                a.dw_blocks = 0;
        }
        switch (mt) {
        case 1: e = chunk_launch<1>(c, s); break;
        case 2: e = chunk_launch<2>(c, s); break;
        case 3: e = chunk_launch<3>(c, s); break;
        default: e = chunk_launch<4>(c, s); break;
        }
    }
    return e;
}

hipError_t launch_linear_backward(const LinearDesc& d, const uint16_t* dy, int64_t M, uint16_t* dx, float* dw,
                                  void* ws, const BwdPlan& p, hipStream_t s)
{
    return launch_linear_backward_batched(&d, &dy, 1, M, &dx, &dw, &ws, &p, s);
}

}  // namespace owq
