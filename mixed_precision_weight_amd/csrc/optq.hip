// optq.hip -- OPTQ with the weak columns last (gfx950).
//
// OWQ quantises the dense columns with OPTQ's sequential, column-by-column
// quantisation and error compensation; the weak columns are moved to the end so
// that their fp16 values absorb compensation without being quantised, and the
// Hessian 2 X^T X is the one the weak-column selection uses ([PL] "OPTQ: Weight
// Quantization for LLMs" pp.2-3, "OWQ: Outlier-aware Weight Quantization" p.4,
// "Quantization efficiency" (paper "Quantization Speed" p.7); [PL] =
// paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for Efficient
// Fine-Tuning and Inference of Large Language Models"). The steps:
//   H = 2 X^T X (fp64), a zero diagonal entry set to 1, then 1 % of the mean
//   diagonal added to it; columns in the order dense (ascending), weak
//   (ascending); in that order taken backwards, H = L L^T (Cholesky) and
//   U = reverse(L^-1), the upper-triangular factor with H^-1 = U^T U; each row is
//   quantised column by column with its min-max step and zero point, the error
//   e = (w - s (q - z)) / U_aa of a column updating each later column b by
//   e U_ab, in batches of 128 columns (inside a batch column by column, the later
//   batches once per batch with the sum over the batch in column order); the weak
//   block is the compensated weak weights rounded to fp16.
//
// Every sum runs in the same order as that definition (one thread per output,
// sequential), so codes, steps, zero points and the weak block are bitwise the
// oracle's. The kernels are plain vector-ALU fp64 code. The Cholesky factor and
// the triangular inverse are blocked (a panel solve, then an update of
// everything right of / below it) with every entry's running sum kept in the
// definition's order: the blocking only decides when each term is added, not in
// which order.
//
// Built with -ffp-contract=off: products and sums are separately rounded as in
// the definition.
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

constexpr int kOptqBatch = 128;

constexpr int kSlotO[32] = {1,  6,  2,  7,  3,  8,  4,  9,  5,  10, 11, 16, 12, 17, 13, 18,
                            14, 19, 15, 20, 21, 26, 22, 27, 23, 28, 24, 29, 25, 30, 0,  31};

__device__ __forceinline__ int weak_before_dense_o(const int32_t* __restrict__ idx, int k, int p)
{
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] - mid <= p)
            lo = mid + 1;
        else
            hi = mid;
    }
    return lo;
}

// perm[a]: the column at position a (dense ascending, then weak ascending);
// invr[j]: the position of column j in the reversed order (K - 1 - a)
__global__ void k_optq_perm(const int32_t* __restrict__ idx, int k, int K, int32_t* __restrict__ perm,
                            int32_t* __restrict__ invr)
{
    const int a = blockIdx.x * 256 + threadIdx.x;
    if (a >= K)
        return;
    const int Kd = K - k;
    const int j = a < Kd ? a + weak_before_dense_o(idx, k, a) : idx[a - Kd];
    perm[a] = j;
    invr[j] = K - 1 - a;
}

// Hr[a][b] = 2 sum_t X[t][rp(a)] X[t][rp(b)] for b <= a, rp(a) = perm[K-1-a];
// 64 x 64 output tiles on or below the diagonal, X columns staged in LDS 16
// tokens at a time, each output summed over t in order (the products are exact)
__global__ __launch_bounds__(256) void k_optq_gram(const uint16_t* __restrict__ X, int T, int K,
                                                   const int32_t* __restrict__ perm, double* __restrict__ Hr)
{
    constexpr int TT = 16;
    __shared__ double xa[TT][64], xb[TT][64];
    const int ta = blockIdx.y, tb = blockIdx.x;
    if (tb > ta)
        return;
    const int tid = threadIdx.x;
    const int ra = tid / 16, rb = tid % 16;  // 4 x 4 outputs per thread
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
            acc[i][j] = 0.0;
    for (int t0 = 0; t0 < T; t0 += TT) {
        __syncthreads();
        for (int e = tid; e < TT * 64; e += 256) {
            const int tt = e / 64, c = e % 64;
            const int t = t0 + tt;
            const int a = ta * 64 + c, b = tb * 64 + c;
            xa[tt][c] = (t < T && a < K) ? (double)h2f(X[(int64_t)t * K + perm[K - 1 - a]]) : 0.0;
            xb[tt][c] = (t < T && b < K) ? (double)h2f(X[(int64_t)t * K + perm[K - 1 - b]]) : 0.0;
        }
        __syncthreads();
        const int tn = min(TT, T - t0);
        for (int tt = 0; tt < tn; tt++)
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++)
                    acc[i][j] += xa[tt][ra * 4 + i] * xb[tt][rb * 4 + j];
    }
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int a = ta * 64 + ra * 4 + i, b = tb * 64 + rb * 4 + j;
            if (a < K && b <= a)
                Hr[(int64_t)a * K + b] = 2.0 * acc[i][j];
        }
}

// the diagonal: zero entries become 1, then 1 % of the mean (summed in column
// order by one thread, from LDS chunks that all threads load) is added to each
__global__ __launch_bounds__(1024) void k_optq_diag(double* __restrict__ Hr, int K, const int32_t* __restrict__ invr)
{
    constexpr int CH = 4096;
    __shared__ double dv[CH];
    __shared__ double sh_damp;
    double sum = 0.0;  // thread 0's running sum
    for (int j0 = 0; j0 < K; j0 += CH) {
        const int n = min(CH, K - j0);
        for (int t = threadIdx.x; t < n; t += 1024) {
            const int64_t a = invr[j0 + t];
            double v = Hr[a * K + a];
            if (v == 0.0)
                v = 1.0;
            Hr[a * K + a] = v;
            dv[t] = v;
        }
        __syncthreads();
        if (threadIdx.x == 0)
            for (int t = 0; t < n; t++)
                sum += dv[t];
        __syncthreads();
    }
    if (threadIdx.x == 0)
        sh_damp = 0.01 * (sum / (double)K);
    __syncthreads();
    const double damp = sh_damp;
    for (int j = threadIdx.x; j < K; j += 1024) {
        const int64_t a = invr[j];
        Hr[a * K + a] += damp;
    }
}

// The Cholesky factor in place of the Hessian (lower triangle, row-major), in
// panels of kCholPanel columns. Each entry's value is its Hessian entry minus
// the products L[i][q] L[j][q] for q = 0, 1, ..., j-1, subtracted one at a time
// in that order and then, below the diagonal, divided by L[j][j]: the products
// of the panels to the left are subtracted by k_optq_chol_trail (one panel at a
// time, q ascending inside it), those of the entry's own panel by
// k_optq_chol_diag / k_optq_chol_panel. Every entry thus sees the same
// subtractions in the same order as the column-by-column definition.
constexpr int kCholPanel = 64;

// the panel's diagonal block [q0, q0 + nb)^2, a thread per row, column by column
__global__ __launch_bounds__(64) void k_optq_chol_diag(double* __restrict__ A, int K, int q0)
{
    __shared__ double d[kCholPanel][kCholPanel + 1];
    const int r = threadIdx.x;
    const int nb = min(kCholPanel, K - q0);
    if (r < nb)
        for (int c = 0; c <= r; c++)
            d[r][c] = A[(int64_t)(q0 + r) * K + q0 + c];
    __syncthreads();
    for (int j = 0; j < nb; j++) {
        if (r == j) {
            double v = d[j][j];
            for (int q = 0; q < j; q++)
                v -= d[j][q] * d[j][q];
            d[j][j] = sqrt(v);
        }
        __syncthreads();
        if (r > j && r < nb) {
            double v = d[r][j];
            for (int q = 0; q < j; q++)
                v -= d[r][q] * d[j][q];
            d[r][j] = v / d[j][j];
        }
        __syncthreads();
    }
    if (r < nb)
        for (int c = 0; c <= r; c++)
            A[(int64_t)(q0 + r) * K + q0 + c] = d[r][c];
}

// the panel's rows below its diagonal block (a full panel): a thread per row,
// the row's kCholPanel entries in registers, column by column
__global__ __launch_bounds__(256) void k_optq_chol_panel(double* __restrict__ A, int K, int q0)
{
    __shared__ double d[kCholPanel][kCholPanel + 1];
    for (int e = threadIdx.x; e < kCholPanel * kCholPanel; e += 256) {
        const int r = e / kCholPanel, c = e % kCholPanel;
        d[r][c] = c <= r ? A[(int64_t)(q0 + r) * K + q0 + c] : 0.0;
    }
    __syncthreads();
    const int i = q0 + kCholPanel + blockIdx.x * 256 + threadIdx.x;
    if (i >= K)
        return;
    double* __restrict__ ai = A + (int64_t)i * K + q0;
    double row[kCholPanel];
#pragma unroll
    for (int c = 0; c < kCholPanel; c++)
        row[c] = ai[c];
#pragma unroll
    for (int j = 0; j < kCholPanel; j++) {
        double v = row[j];
#pragma unroll
        for (int q = 0; q < j; q++)
            v -= row[q] * d[j][q];
        row[j] = v / d[j][j];
    }
#pragma unroll
    for (int c = 0; c < kCholPanel; c++)
        ai[c] = row[c];
}

// the entries right of and below the panel [q0, q1): A[i][j] -= L[i][q] L[j][q]
// for q = q0 .. q1-1 in order, i >= j >= q1; 64 x 64 tiles on or below the
// diagonal, 4 x 4 entries per thread, the panel's rows staged in LDS (q-major)
__global__ __launch_bounds__(256) void k_optq_chol_trail(double* __restrict__ A, int K, int q0)
{
    const int q1 = q0 + kCholPanel;
    const int ti = blockIdx.y, tj = blockIdx.x;
    if (tj > ti)
        return;
    __shared__ double li[kCholPanel][64], lj[kCholPanel][64];
    const int i0 = q1 + ti * 64, j0 = q1 + tj * 64;
    for (int e = threadIdx.x; e < 64 * kCholPanel; e += 256) {
        const int r = e / kCholPanel, q = e % kCholPanel;
        li[q][r] = i0 + r < K ? A[(int64_t)(i0 + r) * K + q0 + q] : 0.0;
        lj[q][r] = j0 + r < K ? A[(int64_t)(j0 + r) * K + q0 + q] : 0.0;
    }
    __syncthreads();
    const int ra = threadIdx.x >> 4, rb = threadIdx.x & 15;
    double acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++) {
            const int i = i0 + ra * 4 + x, j = j0 + rb * 4 + y;
            acc[x][y] = (i < K && j <= i) ? A[(int64_t)i * K + j] : 0.0;
        }
#pragma unroll 2
    for (int q = 0; q < kCholPanel; q++) {
        double a4[4], b4[4];
#pragma unroll
        for (int x = 0; x < 4; x++)
            a4[x] = li[q][ra * 4 + x];
#pragma unroll
        for (int y = 0; y < 4; y++)
            b4[y] = lj[q][rb * 4 + y];
#pragma unroll
        for (int x = 0; x < 4; x++)
#pragma unroll
            for (int y = 0; y < 4; y++)
                acc[x][y] -= a4[x] * b4[y];
    }
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++) {
            const int i = i0 + ra * 4 + x, j = j0 + rb * 4 + y;
            if (i < K && j <= i)
                A[(int64_t)i * K + j] = acc[x][y];
        }
}

// L^-1 (row-major, upper part zero; Mi starts as zeros), in row blocks of
// kInvBlock. Entry (i, j), i > j, is -(sum over q = j .. i-1 of L[i][q] Mi[q][j])
// / L[i][i] with the sum taken in ascending q from +0: the terms of the blocks
// above row i's own are added into Mi[i][j] by k_optq_inv_trail (one block at a
// time, q ascending inside it), those of its own block by k_optq_inv_block. The
// terms with q < j are exact zeros (Mi[q][j] = 0) that leave the running sum at
// +0, so the sum is the definition's, term for term.
constexpr int kInvBlock = 32;

// rows [q0, q0 + nb) of L^-1: a thread per column j < q0 + nb, the block's rows
// in order, their values in registers
__global__ __launch_bounds__(256) void k_optq_inv_block(const double* __restrict__ L, double* __restrict__ Mi, int K,
                                                        int q0)
{
    __shared__ double d[kInvBlock][kInvBlock + 1];
    const int nb = min(kInvBlock, K - q0);
    for (int e = threadIdx.x; e < kInvBlock * kInvBlock; e += 256) {
        const int r = e / kInvBlock, c = e % kInvBlock;
        d[r][c] = (r < nb && c <= r) ? L[(int64_t)(q0 + r) * K + q0 + c] : 1.0;
    }
    __syncthreads();
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= q0 + nb)
        return;
    double m[kInvBlock];
#pragma unroll
    for (int r = 0; r < kInvBlock; r++) {
        const int i = q0 + r;
        double v = 0.0;
        if (r < nb && j <= i) {
            if (j == i) {
                v = 1.0 / d[r][r];
            } else {
                double acc = Mi[(int64_t)i * K + j];
#pragma unroll
                for (int c = 0; c < r; c++)
                    acc += d[r][c] * m[c];
                v = -acc / d[r][r];
            }
            Mi[(int64_t)i * K + j] = v;
        }
        m[r] = v;
    }
}

// rows i >= q1 = q0 + kInvBlock, columns j < q1: Mi[i][j] += L[i][q] Mi[q][j] for
// q = q0 .. q1-1 in order; 64 x 64 tiles, 4 x 4 entries per thread
__global__ __launch_bounds__(256) void k_optq_inv_trail(const double* __restrict__ L, double* __restrict__ Mi, int K,
                                                        int q0)
{
    const int q1 = q0 + kInvBlock;
    __shared__ double lb[kInvBlock][64], mb[kInvBlock][64];
    const int i0 = q1 + blockIdx.y * 64, j0 = blockIdx.x * 64;
    for (int e = threadIdx.x; e < 64 * kInvBlock; e += 256) {
        const int r = e / kInvBlock, q = e % kInvBlock;
        lb[q][r] = i0 + r < K ? L[(int64_t)(i0 + r) * K + q0 + q] : 0.0;
        const int qq = e / 64, c = e % 64;
        mb[qq][c] = j0 + c < q1 ? Mi[(int64_t)(q0 + qq) * K + j0 + c] : 0.0;
    }
    __syncthreads();
    const int ra = threadIdx.x >> 4, rb = threadIdx.x & 15;
    double acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++) {
            const int i = i0 + ra * 4 + x, j = j0 + rb * 4 + y;
            acc[x][y] = (i < K && j < q1) ? Mi[(int64_t)i * K + j] : 0.0;
        }
#pragma unroll 2
    for (int q = 0; q < kInvBlock; q++) {
        double a4[4], b4[4];
#pragma unroll
        for (int x = 0; x < 4; x++)
            a4[x] = lb[q][ra * 4 + x];
#pragma unroll
        for (int y = 0; y < 4; y++)
            b4[y] = mb[q][rb * 4 + y];
#pragma unroll
        for (int x = 0; x < 4; x++)
#pragma unroll
            for (int y = 0; y < 4; y++)
                acc[x][y] += a4[x] * b4[y];
    }
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++) {
            const int i = i0 + ra * 4 + x, j = j0 + rb * 4 + y;
            if (i < K && j < q1)
                Mi[(int64_t)i * K + j] = acc[x][y];
        }
}

// zero fill (the upper part of L^-1 must read as exact zeros)
__global__ __launch_bounds__(256) void k_optq_zero(double* __restrict__ p, int64_t n)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < n)
        p[e] = 0.0;
}

// U[a][b] = Mi[K-1-a][K-1-b]
__device__ __forceinline__ double u_at(const double* __restrict__ Mi, int K, int a, int b)
{
    return Mi[(int64_t)(K - 1 - a) * K + (K - 1 - b)];
}

// the working copy: Wc[i][a] = W[i][perm[a]] in fp64
__global__ __launch_bounds__(256) void k_optq_init(const uint16_t* __restrict__ W, int N, int K,
                                                   const int32_t* __restrict__ perm, double* __restrict__ Wc)
{
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)N * K)
        return;
    const int64_t i = e / K;
    const int a = (int)(e % K);
    Wc[e] = (double)h2f(W[i * K + perm[a]]);
}

// one batch [a0, a1) of every row, column by column: a wave per row, lane l holds
// positions a0 + l and a0 + 64 + l; the batch's block of U in LDS
__global__ __launch_bounds__(1024) void k_optq_batch(double* __restrict__ Wc, int N, int K, int Kd, int a0,
                                                     const double* __restrict__ Mi,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros,
                                                     const int32_t* __restrict__ perm, uint8_t* __restrict__ Qc,
                                                     double* __restrict__ Err)
{
    __shared__ double ub[kOptqBatch][kOptqBatch];
    const int a1 = min(K, a0 + kOptqBatch), nb = a1 - a0;
    const int aq = min(a1, Kd);
    for (int e = threadIdx.x; e < kOptqBatch * kOptqBatch; e += 1024) {
        const int r = e / kOptqBatch, c = e % kOptqBatch;
        ub[r][c] = (r < nb && c < nb && c >= r) ? u_at(Mi, K, a0 + r, a0 + c) : 0.0;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int i = blockIdx.x * 16 + wave; i < N; i += gridDim.x * 16) {
        double w0 = lane < nb ? Wc[(int64_t)i * K + a0 + lane] : 0.0;
        double w1 = lane + 64 < nb ? Wc[(int64_t)i * K + a0 + 64 + lane] : 0.0;
        const double sd = (double)h2f(scales[i]);
        const int z = zeros[i];
        for (int a = a0; a < aq; a++) {
            const int p = a - a0;
            const double wa = __shfl(p < 64 ? w0 : w1, p & 63, 64);
            double r = rint(wa / sd);
            r = r < -8.0 ? -8.0 : (r > 8.0 ? 8.0 : r);
            int q = (int)r + z;
            q = q < 0 ? 0 : (q > 7 ? 7 : q);
            const double e = (wa - sd * (double)(q - z)) / ub[p][p];
            if (lane == 0) {
                Qc[(int64_t)i * K + perm[a]] = (uint8_t)q;
                Err[(int64_t)i * kOptqBatch + p] = e;
            }
            const int b0 = lane, b1 = lane + 64;
            if (b0 > p && b0 < nb)
                w0 -= e * ub[p][b0];
            if (b1 > p && b1 < nb)
                w1 -= e * ub[p][b1];
        }
        if (lane < nb)
            Wc[(int64_t)i * K + a0 + lane] = w0;
        if (lane + 64 < nb)
            Wc[(int64_t)i * K + a0 + 64 + lane] = w1;
    }
}

// the later columns: Wc[i][b] -= sum_{a0 <= a < aq} Err[i][a - a0] U[a][b], the sum
// in column order; a thread per (row, column), 64 columns x 16 rows per block
__global__ __launch_bounds__(256) void k_optq_trail(double* __restrict__ Wc, int N, int K, int a0, int aq, int a1,
                                                    const double* __restrict__ Mi, const double* __restrict__ Err)
{
    __shared__ double uc[kOptqBatch][64];
    __shared__ double er[16][kOptqBatch];
    const int tid = threadIdx.x;
    const int cb = a1 + blockIdx.x * 64;
    const int i0 = blockIdx.y * 16;
    const int na = aq - a0;
    for (int e = tid; e < kOptqBatch * 64; e += 256) {
        const int r = e / 64, c = e % 64;
        uc[r][c] = (r < na && cb + c < K) ? u_at(Mi, K, a0 + r, cb + c) : 0.0;
    }
    for (int e = tid; e < 16 * kOptqBatch; e += 256) {
        const int r = e / kOptqBatch, c = e % kOptqBatch;
        er[r][c] = (i0 + r < N && c < na) ? Err[(int64_t)(i0 + r) * kOptqBatch + c] : 0.0;
    }
    __syncthreads();
    const int c = tid & 63, rg = tid >> 6;  // 4 row groups of 4 rows
    const int b = cb + c;
    if (b >= K)
        return;
    for (int rr = 0; rr < 4; rr++) {
        const int ri = rg * 4 + rr;
        const int i = i0 + ri;
        if (i >= N)
            break;
        double acc = 0.0;
        for (int a = 0; a < na; a++)
            acc += er[ri][a] * uc[a][c];
        Wc[(int64_t)i * K + b] -= acc;
    }
}

// nearest binary16 of a binary64 value (ties to even): round to fp32 with the
// sticky bit kept in the last place (round to odd), then fp32 -> fp16; with 13
// spare bits the second rounding cannot be a double rounding
__device__ __forceinline__ uint16_t f64_to_f16_rne(double d)
{
    float t = (float)d;
    if ((double)t != d) {
        uint32_t b = __builtin_bit_cast(uint32_t, t);
        if (fabs((double)t) > fabs(d))
            b -= 1;  // rounded away from zero: step back toward it
        b |= 1u;
        t = __builtin_bit_cast(float, b);
    }
    return f2h(t);
}

// codes -> latency-favoured groups (weak columns: the zero point), and the weak
// block from the compensated weak weights
__global__ __launch_bounds__(256) void k_optq_finish(const uint8_t* __restrict__ Qc, const double* __restrict__ Wc,
                                                     int N, int K, int Kd, const int32_t* __restrict__ idx, int k,
                                                     const uint8_t* __restrict__ zeros, uint32_t* __restrict__ q,
                                                     uint16_t* __restrict__ ww)
{
    const int G = K >> 5;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)N * G)
        return;
    const int64_t i = e / G;
    const int g = (int)(e % G);
    const uint32_t z = zeros[i];
    // which columns of this group are weak: binary search for the first weak
    // index >= 32 g, then walk
    int lo = 0, hi = k;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (idx[mid] < 32 * g)
            lo = mid + 1;
        else
            hi = mid;
    }
    uint32_t o[3] = {0u, 0u, 0u};
    int c = lo;
    for (int cc = 0; cc < 32; cc++) {
        const int j = 32 * g + cc;
        uint32_t cd;
        if (c < k && idx[c] == j) {
            cd = z;
            c++;
        } else {
            cd = Qc[i * K + j];
        }
        const int pos = 3 * kSlotO[cc], wd = pos >> 5, off = pos & 31;
        o[wd] |= cd << off;
        if (off > 29)
            o[wd + 1] |= cd >> (32 - off);
    }
    uint32_t* dst = q + (i * G + g) * 3;
    dst[0] = o[0];
    dst[1] = o[1];
    dst[2] = o[2];
    if (g == 0)
        for (int cw = 0; cw < k; cw++)
            ww[i * k + cw] = f64_to_f16_rne(Wc[i * K + Kd + cw]);
}

size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

OptqPlan optq_plan(int64_t N, int64_t K, int32_t k)
{
    (void)k;
    OptqPlan p;
    size_t o = 0;
    p.off_perm = o;
    o = al256(o + (size_t)K * sizeof(int32_t));
    p.off_invr = o;
    o = al256(o + (size_t)K * sizeof(int32_t));
    p.off_h = o;  // the Hessian, factored in place into L
    o = al256(o + (size_t)K * K * sizeof(double));
    p.off_mi = o;  // L^-1
    o = al256(o + (size_t)K * K * sizeof(double));
    p.off_wc = o;
    o = al256(o + (size_t)N * K * sizeof(double));
    p.off_err = o;
    o = al256(o + (size_t)N * kOptqBatch * sizeof(double));
    p.off_qc = o;
    o = al256(o + (size_t)N * K);
    p.total = o;
    return p;
}

hipError_t launch_pack_optq(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            const int32_t* idx, int32_t k, uint32_t* q, uint16_t* scales, uint8_t* zeros,
                            uint16_t* ww, void* ws, const OptqPlan& p, hipStream_t s)
{
    char* base = static_cast<char*>(ws);
    int32_t* perm = reinterpret_cast<int32_t*>(base + p.off_perm);
    int32_t* invr = reinterpret_cast<int32_t*>(base + p.off_invr);
    double* Hr = reinterpret_cast<double*>(base + p.off_h);  // H, then L
    double* Mi = reinterpret_cast<double*>(base + p.off_mi);
    double* Wc = reinterpret_cast<double*>(base + p.off_wc);
    double* Err = reinterpret_cast<double*>(base + p.off_err);
    uint8_t* Qc = reinterpret_cast<uint8_t*>(base + p.off_qc);
    const int Ki = (int)K, Ni = (int)N, Kd = (int)(K - k);

    // the steps and zero points (the min-max fit of the dense columns) and the
    // weak block's place: the latency-favoured pack
    hipError_t e = launch_pack(W, N, K, idx, k, q, scales, zeros, ww, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(k_optq_perm, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, idx, (int)k, Ki, perm, invr);
    const unsigned tiles = (unsigned)((K + 63) / 64);
    hipLaunchKernelGGL(k_optq_gram, dim3(tiles, tiles), dim3(256), 0, s, X, (int)T, Ki, perm, Hr);
    hipLaunchKernelGGL(k_optq_diag, dim3(1), dim3(1024), 0, s, Hr, Ki, invr);
    for (int q0 = 0; q0 < Ki; q0 += kCholPanel) {
        hipLaunchKernelGGL(k_optq_chol_diag, dim3(1), dim3(64), 0, s, Hr, Ki, q0);
        const int rest = Ki - q0 - kCholPanel;
        if (rest > 0) {
            hipLaunchKernelGGL(k_optq_chol_panel, dim3((unsigned)((rest + 255) / 256)), dim3(256), 0, s, Hr, Ki, q0);
            const unsigned nt = (unsigned)((rest + 63) / 64);
            hipLaunchKernelGGL(k_optq_chol_trail, dim3(nt, nt), dim3(256), 0, s, Hr, Ki, q0);
        }
    }
    hipLaunchKernelGGL(k_optq_zero, dim3((unsigned)((K * K + 255) / 256)), dim3(256), 0, s, Mi, K * K);
    for (int q0 = 0; q0 < Ki; q0 += kInvBlock) {
        const int q1 = q0 + kInvBlock < Ki ? q0 + kInvBlock : Ki;
        hipLaunchKernelGGL(k_optq_inv_block, dim3((unsigned)((q1 + 255) / 256)), dim3(256), 0, s, Hr, Mi, Ki, q0);
        if (q1 < Ki)
            hipLaunchKernelGGL(k_optq_inv_trail, dim3((unsigned)((q1 + 63) / 64), (unsigned)((Ki - q1 + 63) / 64)),
                               dim3(256), 0, s, Hr, Mi, Ki, q0);
    }
    hipLaunchKernelGGL(k_optq_init, dim3((unsigned)((N * K + 255) / 256)), dim3(256), 0, s, W, Ni, Ki, perm, Wc);
    const unsigned rows_blocks = (unsigned)((N + 15) / 16);
    for (int a0 = 0; a0 < Kd; a0 += kOptqBatch) {
        const int a1 = a0 + kOptqBatch < Ki ? a0 + kOptqBatch : Ki;
        const int aq = a1 < Kd ? a1 : Kd;
        hipLaunchKernelGGL(k_optq_batch, dim3(rows_blocks < 4096 ? rows_blocks : 4096), dim3(1024), 0, s, Wc, Ni, Ki,
                           Kd, a0, Mi, scales, zeros, perm, Qc, Err);
        if (a1 < Ki)
            hipLaunchKernelGGL(k_optq_trail, dim3((unsigned)((K - a1 + 63) / 64), rows_blocks), dim3(256), 0, s, Wc,
                               Ni, Ki, a0, aq, a1, Mi, Err);
    }
    const int64_t G = K / 32;
    hipLaunchKernelGGL(k_optq_finish, dim3((unsigned)((N * G + 255) / 256)), dim3(256), 0, s, Qc, Wc, Ni, Ki, Kd,
                       idx, (int)k, zeros, q, ww);
    return hipGetLastError();
}

}  // namespace owq
