/*
 * owq_oracle.c -- plain, slow CPU oracle of the OWQ hot path.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load it; the GPU library never does, and
 * the two share no source. Built with gcc -O2 -ffp-contract=off (no fused
 * multiply-add, no fast-math), so every fp32 step below is one IEEE binary32
 * operation rounded to nearest-even, and every sum is an fp64 sum in loop order.
 * OpenMP only spreads independent outputs over threads (owq_oracle_linear_rows);
 * it never splits a sum.
 *
 * Pages cited (see owq_oracle.h for the full titles):
 *   [PL] paperlayer.ai notes on the OWQ paper, by section heading.
 *   [EL] research.elamur.ai summary of the OWQ paper, by section heading.
 *
 * Readings taken where the pages are silent (each is also listed in the design
 * notes of the repository):
 *   R1  the min-max range always contains 0 (lo = min(0, min w), hi = max(0, max w)),
 *       so the zero point is itself a valid 3-bit code;
 *   R2  a row with hi == lo, or whose fp32 step rounds to fp16 zero, gets step 1.0
 *       and zero point 0 (every code is then the zero point's neighbourhood: 0);
 *   R3  step s32 = (hi - lo) / 7 in fp32, stored as fp16 (nearest-even); the stored
 *       fp16 value is the one used for quantising and dequantising;
 *   R4  "nearest rounding" is round-half-to-even; code = clamp(rint(w / s) + z, 0, 7)
 *       (round first, then add the integer zero point), IEEE division;
 *   R5  the score uses the round-to-nearest error of a full-row fit (no weak set
 *       exists yet); the pack fits each row on its dense (non-weak) columns only;
 *   R6  score ties are broken by the lower column index; the weak indices and the
 *       weak columns are stored in ascending column order;
 *   R7  bit layout: a 32-column group is one 96-bit word w0|w1<<32|w2<<64 of 32
 *       three-bit slots, slot s at bits [3s, 3s+3); column c of the group is
 *       stored in slot kSlot[c]: columns 2p and 2p+1 take the p-th slot pair
 *       (1,6) (2,7) (3,8) (4,9) (5,10) (11,16) (12,17) (13,18) (14,19) (15,20)
 *       (21,26) (22,27) (23,28) (24,29) (25,30) (0,31). The pages fix only that
 *       32 codes fill 3 uint32 along K.
 */
#include "owq_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- fp16 ---- */

/* IEEE 754 binary16: sign bit, 5-bit biased exponent (bias 15), 10-bit fraction.
 * Exponent 0 encodes subnormals m * 2^-24; exponent 31 encodes inf / NaN. */
double owq_oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* Nearest binary16 to a binary32 value, ties to even. The scaled value below is
 * exact in binary64 (power-of-two scaling), so rint() performs exactly the
 * round-half-to-even step of the definition. */
uint16_t owq_oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs((double)f);
    if (isnan(f))
        return sign | 0x7e00;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 and above: infinity */
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) { /* subnormal range, quantum 2^-24 */
        double q = rint(ldexp(a, 24));
        return sign | (uint16_t)q; /* q == 1024 is the smallest normal, 0x0400 */
    }
    int e2;
    frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1; /* a in [2^E, 2^(E+1)) */
    double q = rint(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(q - 1024.0);
}

static float f16_to_f32(uint16_t h) { return (float)owq_oracle_f16_to_f64(h); }

/* Nearest binary16 to a binary64 value, ties to even (the same steps as the
 * binary32 conversion, on the exact binary64 value). */
uint16_t owq_oracle_f64_to_f16(double f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    double a = fabs(f);
    if (isnan(f))
        return sign | 0x7e00;
    if (a >= 65520.0)
        return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {
        double m0 = rint(ldexp(a, 24));
        return sign | (uint16_t)m0;
    }
    int e2;
    frexp(a, &e2);
    int E = e2 - 1;
    double m = rint(ldexp(a, 10 - E));
    if (m == 2048.0) {
        m = 1024.0;
        E += 1;
    }
    return sign | (uint16_t)((E + 15) << 10) | (uint16_t)(m - 1024.0);
}

/* ------------------------------------------------------------ quantiser ---- */

/* Min-max round-to-nearest parameters of one output row: step size and zero
 * point of an asymmetric 3-bit grid (2^3 - 1 = 7 steps). The quantiser with a
 * step size and zero point and nearest rounding: [PL] "Low-precision
 * quantization" (paper "Quantization Configuration Search", pp. 4-5); min-max
 * round-to-nearest as the simple quantiser: [EL] "Key points". Readings R1-R4. */
void owq_oracle_qparams(const uint16_t* row, const uint8_t* use, int64_t K,
                        uint16_t* s16, uint8_t* z)
{
    float lo = 0.0f, hi = 0.0f; /* R1 */
    for (int64_t j = 0; j < K; j++) {
        if (use && !use[j])
            continue;
        float w = f16_to_f32(row[j]);
        if (w < lo)
            lo = w;
        if (w > hi)
            hi = w;
    }
    if (hi == lo) { /* R2 */
        *s16 = 0x3c00;
        *z = 0;
        return;
    }
    float s32 = (hi - lo) / 7.0f;
    uint16_t s = owq_oracle_f32_to_f16(s32); /* R3 */
    if ((s & 0x7fff) == 0) {                 /* R2: step below half the smallest fp16 */
        *s16 = 0x3c00;
        *z = 0;
        return;
    }
    float sf = f16_to_f32(s);
    float zr = rintf(-lo / sf); /* R4 */
    int zi = zr < 0.0f ? 0 : zr > 7.0f ? 7 : (int)zr;
    *s16 = s;
    *z = (uint8_t)zi;
}

/* code = clamp(rint(w / s) + z, 0, 7) (R4). The intermediate clamp to [-8, 8]
 * only keeps the float-to-int conversion defined: any r beyond it already
 * saturates the final clamp for every z in [0, 7]. */
int owq_oracle_code(uint16_t w, uint16_t s16, uint8_t z)
{
    float sf = f16_to_f32(s16);
    float r = rintf(f16_to_f32(w) / sf);
    if (r < -8.0f)
        r = -8.0f;
    if (r > 8.0f)
        r = 8.0f;
    int q = (int)r + (int)z;
    return q < 0 ? 0 : q > 7 ? 7 : q;
}

/* ---------------------------------------------------------- calibration ---- */

/* The layer-wise objective ||W X - W^ X||^2 splits into one quadratic error per
 * output row that shares one input-channel Hessian ([PL] "Problem Definition",
 * "Error Decomposition", "Error Analysis", paper p.3 and appendix section 1 p.10).
 * For row i, d^2/dW_i^2 of ||(W_i - W^_i) X^T||^2 is H = 2 X^T X with X as
 * [T][K]; its diagonal is lambda_j = 2 sum_t X[t][j]^2. */
void owq_oracle_hessian_diag(const uint16_t* X, int64_t T, int64_t K, double* lambda)
{
    for (int64_t j = 0; j < K; j++)
        lambda[j] = 0.0;
    for (int64_t t = 0; t < T; t++)
        for (int64_t j = 0; j < K; j++) {
            double v = owq_oracle_f16_to_f64(X[t * K + j]);
            lambda[j] += v * v;
        }
    for (int64_t j = 0; j < K; j++)
        lambda[j] *= 2.0;
}

/* Squared perturbation norm of every column under round-to-nearest of the
 * full row: e_j = sum_i dW_ij^2, dW = W - W^ ([PL] appendix section 1 p.10 defines
 * the row perturbation dW_i = W_i - W^_i). R5: the fit covers all K columns. */
void owq_oracle_rtn_col_err(const uint16_t* W, int64_t N, int64_t K, double* e)
{
    for (int64_t j = 0; j < K; j++)
        e[j] = 0.0;
    for (int64_t i = 0; i < N; i++) {
        const uint16_t* row = W + i * K;
        uint16_t s16;
        uint8_t z;
        owq_oracle_qparams(row, NULL, K, &s16, &z);
        double s = owq_oracle_f16_to_f64(s16);
        for (int64_t j = 0; j < K; j++) {
            int q = owq_oracle_code(row[j], s16, z);
            double d = owq_oracle_f16_to_f64(row[j]) - s * (double)(q - (int)z);
            e[j] += d * d;
        }
    }
}

/* Column sensitivity = Hessian diagonal element times the column's squared
 * perturbation norm ([PL] "Weak-column selection", paper p.4; [EL] "Interesting
 * ideas": scoring by weight error alone was worse). */
void owq_oracle_calibrate_score(const uint16_t* W, int64_t N, int64_t K,
                                const uint16_t* X, int64_t T,
                                double* lambda, double* score)
{
    double* e = (double*)malloc((size_t)K * sizeof(double));
    owq_oracle_hessian_diag(X, T, K, lambda);
    owq_oracle_rtn_col_err(W, N, K, e);
    for (int64_t j = 0; j < K; j++)
        score[j] = lambda[j] * e[j];
    free(e);
}

static const double* g_sort_score; /* comparator context (single-threaded oracle) */

static int cmp_score_desc(const void* a, const void* b)
{
    int32_t ia = *(const int32_t*)a, ib = *(const int32_t*)b;
    double sa = g_sort_score[ia], sb = g_sort_score[ib];
    if (sa > sb)
        return -1;
    if (sa < sb)
        return 1;
    return ia < ib ? -1 : ia > ib ? 1 : 0; /* R6 */
}

static int cmp_int_asc(const void* a, const void* b)
{
    int32_t ia = *(const int32_t*)a, ib = *(const int32_t*)b;
    return ia < ib ? -1 : ia > ib ? 1 : 0;
}

/* Top-k columns by sensitivity become the weak columns ([PL] "Weak-column
 * selection", paper p.4). Sort all columns by (score desc, index asc), keep the
 * first k, return them in ascending order (R6). */
void owq_oracle_select_weak(const double* score, int64_t K, int32_t k, int32_t* weak_idx)
{
    int32_t* order = (int32_t*)malloc((size_t)K * sizeof(int32_t));
    for (int64_t j = 0; j < K; j++)
        order[j] = (int32_t)j;
    g_sort_score = score;
    qsort(order, (size_t)K, sizeof(int32_t), cmp_score_desc);
    memcpy(weak_idx, order, (size_t)k * sizeof(int32_t));
    qsort(weak_idx, (size_t)k, sizeof(int32_t), cmp_int_asc);
    free(order);
}

/* ------------------------------------------------------------------ pack ---- */

/* Slot of column c within its 32-column group (R7). */
static const int kSlot[32] = {1,  6,  2,  7,  3,  8,  4,  9,  5,  10, 11, 16, 12, 17, 13, 18,
                              14, 19, 15, 20, 21, 26, 22, 27, 23, 28, 24, 29, 25, 30, 0,  31};

/* Write the code of column c (3 bits) of one 32-column group into its three
 * words (R7). */
static void put_code(uint32_t* grp, int c, int code)
{
    for (int b = 0; b < 3; b++) {
        int pos = 3 * kSlot[c] + b;
        if ((code >> b) & 1)
            grp[pos / 32] |= (uint32_t)1 << (pos % 32);
    }
}

static int get_code(const uint32_t* grp, int c)
{
    int v = 0;
    for (int b = 0; b < 3; b++) {
        int pos = 3 * kSlot[c] + b;
        v |= (int)((grp[pos / 32] >> (pos % 32)) & 1u) << b;
    }
    return v;
}

/* One row of the latency-favoured storage under the row's (s16, z): codes of
 * the dense columns, the zero point for the weak ones, packed 32 per group. */
static void pack_row(const uint16_t* row, const uint8_t* weak, int64_t G, uint16_t s16, uint8_t z,
                     uint32_t* qrow)
{
    for (int64_t g = 0; g < G; g++) {
        uint32_t* grp = qrow + g * 3;
        grp[0] = grp[1] = grp[2] = 0;
        for (int c = 0; c < 32; c++) {
            int64_t j = g * 32 + c;
            int code = weak[j] ? (int)z : owq_oracle_code(row[j], s16, z);
            put_code(grp, c, code);
        }
    }
}

/* Latency-favoured storage: a complete low-precision matrix whose weak columns
 * are zero-filled, plus the weak columns kept separately in fp16 ([PL] "Storage
 * Methods", appendix section 2 pp.10-11). Weak columns are excluded from
 * quantisation ([PL] "Weak-column selection", p.4), so each row is fitted on its
 * dense columns only (R5); "zero-filled" for an asymmetric grid means the code
 * whose dequantised value is 0, the zero point. */
void owq_oracle_pack(const uint16_t* W, int64_t N, int64_t K,
                     const int32_t* weak_idx, int32_t k,
                     uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                     uint16_t* w_weak)
{
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    uint8_t* dense = (uint8_t*)malloc((size_t)K);
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    for (int64_t j = 0; j < K; j++)
        dense[j] = !weak[j];
    int64_t G = K / 32;
    for (int64_t i = 0; i < N; i++) {
        const uint16_t* row = W + i * K;
        uint16_t s16;
        uint8_t z;
        owq_oracle_qparams(row, dense, K, &s16, &z);
        pack_row(row, weak, G, s16, z, qcodes + i * G * 3);
        scales[i] = s16;
        zeros[i] = z;
        for (int32_t c = 0; c < k; c++)
            w_weak[i * k + c] = row[weak_idx[c]];
    }
    free(weak);
    free(dense);
}

/* --------------------------------------------------- storage-favoured form ---- */

/* The storage-favoured representation keeps only the dense columns' codes (the
 * zero-filled weak columns are removed) next to the fp16 weak columns ([PL]
 * "Storage Methods", appendix section 2 pp.10-11: it drops the unneeded zeros at
 * the price of extra work in the product). Readings: each row's (s16, z) is the
 * latency-favoured pack's (fit over the dense columns, R5); the dense columns'
 * codes follow in ascending column order, 32 to a group in the R7 layout, and the
 * last group of a row is filled up with the zero point (it dequantises to 0).
 * qcodes: [N][ceil((K - k) / 32)][3]. */
void owq_oracle_pack_storage(const uint16_t* W, int64_t N, int64_t K,
                             const int32_t* weak_idx, int32_t k,
                             uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                             uint16_t* w_weak)
{
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    uint8_t* dense = (uint8_t*)malloc((size_t)K);
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    for (int64_t j = 0; j < K; j++)
        dense[j] = !weak[j];
    int64_t Kd = K - k;
    int64_t Gd = (Kd + 31) / 32;
    for (int64_t i = 0; i < N; i++) {
        const uint16_t* row = W + i * K;
        uint16_t s16;
        uint8_t z;
        owq_oracle_qparams(row, dense, K, &s16, &z);
        uint32_t* qrow = qcodes + i * Gd * 3;
        for (int64_t e = 0; e < Gd * 3; e++)
            qrow[e] = 0;
        int64_t p = 0; /* position among the dense columns */
        for (int64_t j = 0; j < K; j++) {
            if (weak[j])
                continue;
            put_code(qrow + (p / 32) * 3, (int)(p % 32), owq_oracle_code(row[j], s16, z));
            p++;
        }
        for (; p < Gd * 32; p++)
            put_code(qrow + (p / 32) * 3, (int)(p % 32), z);
        scales[i] = s16;
        zeros[i] = z;
        for (int32_t c = 0; c < k; c++)
            w_weak[i * k + c] = row[weak_idx[c]];
    }
    free(weak);
    free(dense);
}

/* The product in the storage-favoured form: the dense columns' codes against x
 * at the dense columns (gathered in ascending order), plus the weak columns, in
 * fp64, all tokens of the listed rows (OpenMP over rows). y, bound: [M][R]. */
void owq_oracle_linear_storage_rows(const uint32_t* qcodes, const uint16_t* scales,
                                    const uint8_t* zeros, int64_t N, int64_t K,
                                    const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                    const uint16_t* x, int64_t M,
                                    const int64_t* rows, int64_t R, double* y, double* bound,
                                    int threads)
{
    (void)N;
    int64_t Kd = K - k;
    int64_t Gd = (Kd + 31) / 32;
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    int64_t* dcol = (int64_t*)malloc((size_t)(Kd > 0 ? Kd : 1) * sizeof(int64_t));
    int64_t p = 0;
    for (int64_t j = 0; j < K; j++)
        if (!weak[j])
            dcol[p++] = j;
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 4)
    for (int64_t r = 0; r < R; r++) {
        int64_t i = rows[r];
        double s = owq_oracle_f16_to_f64(scales[i]);
        int z = zeros[i];
        for (int64_t m = 0; m < M; m++) {
            const uint16_t* xm = x + m * K;
            double acc = 0.0, bnd = 0.0;
            for (int64_t q = 0; q < Kd; q++) {
                int code = get_code(qcodes + (i * Gd + q / 32) * 3, (int)(q % 32));
                double t = s * (double)(code - z) * owq_oracle_f16_to_f64(xm[dcol[q]]);
                acc += t;
                bnd += fabs(t);
            }
            for (int32_t c = 0; c < k; c++) {
                double tw = owq_oracle_f16_to_f64(w_weak[i * k + c]) * owq_oracle_f16_to_f64(xm[(size_t)weak_idx[c]]);
                acc += tw;
                bnd += fabs(tw);
            }
            y[m * R + r] = acc;
            bound[m * R + r] = bnd;
        }
    }
    free(dcol);
    free(weak);
}

/* ------------------------------------------------ weak-column tuning: backward ---- */

/* Weak Column Tuning trains only the fp16 weak columns and keeps the 3-bit dense
 * matrix frozen ([PL] "Weak Column Tuning" (paper "PEFT with Weak Column Tuning",
 * p.5); the trainable block is N x k: "Learnable Parameters", appendix section 3,
 * p.13). For y = x W^T with W the dequantised dense matrix (0 at the weak
 * columns) plus the weak columns, and an upstream gradient dy [M][N]:
 *   dx[m][j]      = sum_i dy[m][i] W[i][j]          (the gradient to the layer input)
 *   dw_weak[i][c] = sum_m dy[m][i] x[m][idx_c]      (the gradient of the weak block)
 * in fp64 from the packed bytes; the bounds are the sums of the terms' absolute
 * values. dx, dx_bound: [M][K]; dw, dw_bound: [N][k]. Either pair may be NULL.
 * OpenMP over columns (dx) and rows (dw); each output is one sum in index order. */
void owq_oracle_linear_backward(const uint32_t* qcodes, const uint16_t* scales,
                                const uint8_t* zeros, int64_t N, int64_t K,
                                const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                const uint16_t* x, const uint16_t* dy, int64_t M,
                                double* dx, double* dx_bound, double* dw, double* dw_bound,
                                int threads)
{
    int64_t G = K / 32;
    int nt = threads > 0 ? threads : omp_get_max_threads();
    if (dx) {
        /* the whole matrix W once, row-major, in fp64 */
        double* Wf = (double*)malloc((size_t)(N * K) * sizeof(double));
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = 0; i < N; i++) {
            double s = owq_oracle_f16_to_f64(scales[i]);
            int z = zeros[i];
            for (int64_t j = 0; j < K; j++)
                Wf[i * K + j] = s * (double)(get_code(qcodes + (i * G + j / 32) * 3, (int)(j % 32)) - z);
            for (int32_t c = 0; c < k; c++)
                Wf[i * K + weak_idx[c]] += owq_oracle_f16_to_f64(w_weak[i * k + c]);
        }
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
        for (int64_t j = 0; j < K; j++)
            for (int64_t m = 0; m < M; m++) {
                double acc = 0.0, bnd = 0.0;
                for (int64_t i = 0; i < N; i++) {
                    double t = owq_oracle_f16_to_f64(dy[m * N + i]) * Wf[i * K + j];
                    acc += t;
                    bnd += fabs(t);
                }
                dx[m * K + j] = acc;
                dx_bound[m * K + j] = bnd;
            }
        free(Wf);
    }
    if (dw) {
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
        for (int64_t i = 0; i < N; i++)
            for (int32_t c = 0; c < k; c++) {
                double acc = 0.0, bnd = 0.0;
                for (int64_t m = 0; m < M; m++) {
                    double t = owq_oracle_f16_to_f64(dy[m * N + i]) *
                               owq_oracle_f16_to_f64(x[m * K + weak_idx[c]]);
                    acc += t;
                    bnd += fabs(t);
                }
                dw[i * k + c] = acc;
                dw_bound[i * k + c] = bnd;
            }
    }
}

/* ------------------------------------------ OPTQ with the weak columns last ---- */

/* OWQ quantises the dense columns with OPTQ's sequential column-by-column
 * quantisation and error compensation, the weak columns moved to the end so that
 * their full-precision values absorb compensation without being quantised; the
 * Hessian 2 X^T X is shared with the weak-column selection ([PL] "OPTQ: Weight
 * Quantization for LLMs" (pp.2-3), "OWQ: Outlier-aware Weight Quantization"
 * (p.4), "Quantization efficiency" (paper "Quantization Speed", p.7), "B
 * Experiment Details" (p.10): built on the OPTQ codebase). Readings (the pages
 * give none of these):
 *   P1 H = 2 X^T X in fp64; a column with H_jj == 0 gets H_jj = 1; every H_jj then
 *      gains 1 % of the mean diagonal (damping);
 *   P2 column order: the dense columns ascending, then the weak columns ascending;
 *   P3 the compensation uses U, the upper-triangular factor with H^-1 = U^T U:
 *      the inverse of the Cholesky factor of H taken in reversed column order
 *      (H in reversed order = L L^T, then U reversed back from L^-1);
 *   P4 each row's (step, zero point) is the min-max fit of its original dense
 *      weights (R1-R5); a column's code is clamp(rint(w / s) + z, 0, 7) on the
 *      compensated fp64 weight with an fp64 quotient; its error
 *      e = (w - s (q - z)) / U_aa updates every later column b by e U_ab;
 *   P5 lazy batches of 128 columns: inside a batch the updates are applied column
 *      by column; the later batches get, per column, the sum over the batch's
 *      quantised columns of e U_ab in ascending order, subtracted once;
 *   P6 the weak block is the fp16 rounding (nearest-even) of the compensated weak
 *      weights; weak codes are the zero point (latency-favoured format). */
#define OWQ_OPTQ_BLOCK 128

static int cmp_i32(const void* a, const void* b)
{
    int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
    return x < y ? -1 : x > y ? 1 : 0;
}

/* U (upper, [K][K] row-major, lower part 0) of P3 from the damped, permuted H. */
static void optq_factor(const double* Hp, int64_t K, double* U, int nt)
{
    double* Hr = (double*)malloc((size_t)(K * K) * sizeof(double));
    double* L = (double*)calloc((size_t)(K * K), sizeof(double));
    double* Mi = (double*)calloc((size_t)(K * K), sizeof(double));
    for (int64_t a = 0; a < K; a++)
        for (int64_t b = 0; b < K; b++)
            Hr[a * K + b] = Hp[(K - 1 - a) * K + (K - 1 - b)];
    /* Cholesky Hr = L L^T, column by column */
    for (int64_t j = 0; j < K; j++) {
        double d = Hr[j * K + j];
        for (int64_t q = 0; q < j; q++)
            d -= L[j * K + q] * L[j * K + q];
        double ljj = sqrt(d);
        L[j * K + j] = ljj;
#pragma omp parallel for num_threads(nt) schedule(static)
        for (int64_t i = j + 1; i < K; i++) {
            double acc = Hr[i * K + j];
            for (int64_t q = 0; q < j; q++)
                acc -= L[i * K + q] * L[j * K + q];
            L[i * K + j] = acc / ljj;
        }
    }
    /* L^-1, column by column, rows downwards; column j of it is kept
     * contiguous (Mi[j][i] = (L^-1)[i][j]) */
#pragma omp parallel for num_threads(nt) schedule(dynamic, 8)
    for (int64_t j = 0; j < K; j++) {
        double* mj = Mi + j * K;
        mj[j] = 1.0 / L[j * K + j];
        for (int64_t i = j + 1; i < K; i++) {
            double acc = 0.0;
            for (int64_t q = j; q < i; q++)
                acc += L[i * K + q] * mj[q];
            mj[i] = -acc / L[i * K + i];
        }
    }
    for (int64_t a = 0; a < K; a++)
        for (int64_t b = 0; b < K; b++)
            U[a * K + b] = b >= a ? Mi[(K - 1 - b) * K + (K - 1 - a)] : 0.0;
    free(Hr);
    free(L);
    free(Mi);
}

void owq_oracle_optq_factor(const uint16_t* X, int64_t T, int64_t K, const int32_t* weak_idx, int32_t k,
                            double* U, int threads)
{
    int nt = threads > 0 ? threads : omp_get_max_threads();
    double* H = (double*)malloc((size_t)(K * K) * sizeof(double));
    /* the columns of X, each contiguous (Xc[j][t] = X[t][j]) */
    double* Xc = (double*)malloc((size_t)(T * K) * sizeof(double));
    for (int64_t t = 0; t < T; t++)
        for (int64_t j = 0; j < K; j++)
            Xc[j * T + t] = owq_oracle_f16_to_f64(X[(size_t)(t * K + j)]);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 4)
    for (int64_t i = 0; i < K; i++)
        for (int64_t j = 0; j < K; j++) {
            double acc = 0.0;
            for (int64_t t = 0; t < T; t++)
                acc += Xc[i * T + t] * Xc[j * T + t];
            H[i * K + j] = 2.0 * acc;
        }
    free(Xc);
    double dsum = 0.0; /* P1 */
    for (int64_t j = 0; j < K; j++) {
        if (H[j * K + j] == 0.0)
            H[j * K + j] = 1.0;
        dsum += H[j * K + j];
    }
    double damp = 0.01 * (dsum / (double)K);
    for (int64_t j = 0; j < K; j++)
        H[j * K + j] += damp;
    /* P2 */
    int32_t* perm = (int32_t*)malloc((size_t)K * sizeof(int32_t));
    int32_t* w = (int32_t*)malloc((size_t)(k > 0 ? k : 1) * sizeof(int32_t));
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    for (int32_t c = 0; c < k; c++) {
        w[c] = weak_idx[c];
        weak[weak_idx[c]] = 1;
    }
    qsort(w, (size_t)k, sizeof(int32_t), cmp_i32);
    int64_t p = 0;
    for (int64_t j = 0; j < K; j++)
        if (!weak[j])
            perm[p++] = (int32_t)j;
    for (int32_t c = 0; c < k; c++)
        perm[p++] = w[c];
    double* Hp = (double*)malloc((size_t)(K * K) * sizeof(double));
    for (int64_t a = 0; a < K; a++)
        for (int64_t b = 0; b < K; b++)
            Hp[a * K + b] = H[(int64_t)perm[a] * K + perm[b]];
    optq_factor(Hp, K, U, nt); /* P3 */
    free(Hp);
    free(H);
    free(perm);
    free(w);
    free(weak);
}

/* OPTQ pack: latency-favoured outputs (qcodes, scales, zeros, w_weak) of the
 * sequential quantisation P4-P6 of every row (OpenMP over rows), given U. */
void owq_oracle_optq_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                          const double* U, uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                          uint16_t* w_weak, int threads)
{
    int nt = threads > 0 ? threads : omp_get_max_threads();
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    uint8_t* dense = (uint8_t*)malloc((size_t)K);
    int32_t* perm = (int32_t*)malloc((size_t)K * sizeof(int32_t));
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    int64_t Kd = 0;
    for (int64_t j = 0; j < K; j++) {
        dense[j] = !weak[j];
        if (!weak[j])
            perm[Kd++] = (int32_t)j;
    }
    for (int32_t c = 0; c < k; c++)
        perm[Kd + c] = weak_idx[c]; /* ascending by the caller's contract */
    int64_t G = K / 32;
#pragma omp parallel num_threads(nt)
    {
        double* wr = (double*)malloc((size_t)K * sizeof(double));
        double* acc = (double*)malloc((size_t)K * sizeof(double));
        double* err = (double*)malloc(OWQ_OPTQ_BLOCK * sizeof(double));
        uint8_t* code = (uint8_t*)malloc((size_t)K);
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < N; i++) {
            const uint16_t* row = W + i * K;
            uint16_t s16;
            uint8_t z;
            owq_oracle_qparams(row, dense, K, &s16, &z); /* P4 */
            double sd = owq_oracle_f16_to_f64(s16);
            for (int64_t a = 0; a < K; a++)
                wr[a] = owq_oracle_f16_to_f64(row[perm[a]]);
            for (int64_t a0 = 0; a0 < K; a0 += OWQ_OPTQ_BLOCK) { /* P5 */
                int64_t a1 = a0 + OWQ_OPTQ_BLOCK < K ? a0 + OWQ_OPTQ_BLOCK : K;
                int64_t aq = a1 < Kd ? a1 : Kd; /* quantised columns of this batch end here */
                for (int64_t a = a0; a < aq; a++) {
                    double r = rint(wr[a] / sd);
                    if (r < -8.0)
                        r = -8.0;
                    if (r > 8.0)
                        r = 8.0;
                    int q = (int)r + (int)z;
                    q = q < 0 ? 0 : q > 7 ? 7 : q;
                    code[perm[a]] = (uint8_t)q;
                    double e = (wr[a] - sd * (double)(q - (int)z)) / U[a * K + a];
                    err[a - a0] = e;
                    for (int64_t b = a + 1; b < a1; b++)
                        wr[b] -= e * U[a * K + b];
                }
                /* per later column b: acc_b = sum over the batch, a ascending
                 * (a outer so that U is read along its rows) */
                for (int64_t b = a1; b < K; b++)
                    acc[b] = 0.0;
                for (int64_t a = a0; a < aq; a++)
                    for (int64_t b = a1; b < K; b++)
                        acc[b] += err[a - a0] * U[a * K + b];
                for (int64_t b = a1; b < K; b++)
                    wr[b] -= acc[b];
            }
            for (int32_t c = 0; c < k; c++) { /* P6 */
                code[weak_idx[c]] = z;
                w_weak[i * k + c] = owq_oracle_f64_to_f16(wr[Kd + c]);
            }
            for (int64_t g = 0; g < G; g++) {
                uint32_t* grp = qcodes + (i * G + g) * 3;
                grp[0] = grp[1] = grp[2] = 0;
                for (int c = 0; c < 32; c++)
                    put_code(grp, c, code[g * 32 + c]);
            }
            scales[i] = s16;
            zeros[i] = z;
        }
        free(wr);
        free(acc);
        free(err);
        free(code);
    }
    free(weak);
    free(dense);
    free(perm);
}

/* ------------------------------------------------- step / zero-point search ---- */

/* Truncation-aware choice of one row's step size and zero point: a 2D grid
 * search over the step size and the zero point, with round-to-nearest codes
 * clamped to the 3-bit range, so that a narrower range than min-max can win by
 * truncating a few large weights ([PL] "Low-precision quantization", paper
 * "Quantization Configuration Search", pp.4-5; the effect on quality is in
 * "Quantization quality", p.5). Readings (the pages give neither the grid nor
 * the objective):
 *   S1 the grid: steps s_a = fp16(s32 * (1 - a/40)) for a = 0 .. steps-1, with
 *      s32 = (hi - lo) / 7 the fp32 min-max step of R1/R3 (a = 0 is the min-max
 *      step itself; the others narrow the range, none widens it; a step that
 *      rounds to fp16 zero is skipped); zero points z = 0 .. 7 (zsearch != 0),
 *      or only the min-max zero point of that step (zsearch == 0);
 *   S2 the objective of a grid point is the row's reconstruction error over its
 *      dense columns, E = sum_j omega_j (w_j - s (code_j - z))^2 with code_j =
 *      clamp(rint(w_j / s) + z, 0, 7) as in R4 and omega_j = lambda_j (the
 *      Hessian diagonal, the output error's diagonal weighting) when lambda is
 *      given, else 1; each term is (d * d), then times lambda_j, added in
 *      ascending column order in fp64;
 *   S3 the smallest E wins; ties go to the smaller a, then the smaller z (the
 *      order the grid is visited in);
 *   S4 a degenerate row (hi == lo, or a min-max step that rounds to fp16 zero)
 *      keeps R2's step 1 and zero point 0.
 * With steps == 1 and zsearch == 0 the grid is the min-max point alone and the
 * result is owq_oracle_qparams'. */
void owq_oracle_search_qparams(const uint16_t* row, const uint8_t* use, int64_t K,
                               const double* lambda, int steps, int zsearch,
                               uint16_t* s16, uint8_t* z)
{
    float lo = 0.0f; /* R1: the range holds 0 */
    float hi = 0.0f;
    for (int64_t j = 0; j < K; j++) {
        if (use && !use[j])
            continue;
        float w = f16_to_f32(row[j]);
        if (w < lo)
            lo = w;
        if (w > hi)
            hi = w;
    }
    *s16 = 0x3c00; /* S4 */
    *z = 0;
    if (hi == lo)
        return;
    float s_mm = (hi - lo) / 7.0f;
    if ((owq_oracle_f32_to_f16(s_mm) & 0x7fff) == 0)
        return;
    /* the dense weights, widened once (exactly) for the grid's many passes */
    int64_t n = 0;
    float* wf = (float*)malloc((size_t)K * sizeof(float));
    double* om = (double*)malloc((size_t)K * sizeof(double));
    for (int64_t j = 0; j < K; j++) {
        if (use && !use[j])
            continue;
        wf[n] = f16_to_f32(row[j]);
        om[n] = lambda ? lambda[j] : 1.0;
        n++;
    }
    double best = INFINITY;
    for (int a = 0; a < steps; a++) {
        float sa32 = s_mm * (1.0f - (float)a / 40.0f); /* S1 */
        uint16_t sa = owq_oracle_f32_to_f16(sa32);
        if ((sa & 0x7fff) == 0)
            continue;
        float sf = f16_to_f32(sa);
        double sd = owq_oracle_f16_to_f64(sa);
        int zmm = 0;
        if (!zsearch) { /* the min-max zero point of this step (R4) */
            float zr = rintf((-lo) / sf);
            zmm = zr < 0.0f ? 0 : zr > 7.0f ? 7 : (int)zr;
        }
        for (int zc = zsearch ? 0 : zmm; zc <= (zsearch ? 7 : zmm); zc++) {
            double E = 0.0; /* S2 */
            for (int64_t e = 0; e < n; e++) {
                /* code = clamp(rint(w / s) + z, 0, 7) (R4), as owq_oracle_code */
                float r = rintf(wf[e] / sf);
                if (r < -8.0f)
                    r = -8.0f;
                if (r > 8.0f)
                    r = 8.0f;
                int q = (int)r + zc;
                q = q < 0 ? 0 : q > 7 ? 7 : q;
                double d = (double)wf[e] - sd * (double)(q - zc);
                double t = d * d;
                if (lambda)
                    t = om[e] * t;
                E += t;
            }
            if (E < best) { /* S3: strict, so the first of equal errors stays */
                best = E;
                *s16 = sa;
                *z = (uint8_t)zc;
            }
        }
    }
    free(wf);
    free(om);
}

/* owq_oracle_pack with each row's (s16, z) from the search above over its dense
 * columns (rows spread over OpenMP threads; threads <= 0: the default). */
void owq_oracle_pack_search(const uint16_t* W, int64_t N, int64_t K,
                            const int32_t* weak_idx, int32_t k, const double* lambda,
                            int steps, int zsearch,
                            uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                            uint16_t* w_weak, int threads)
{
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    uint8_t* dense = (uint8_t*)malloc((size_t)K);
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    for (int64_t j = 0; j < K; j++)
        dense[j] = !weak[j];
    int64_t G = K / 32;
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
    for (int64_t i = 0; i < N; i++) {
        const uint16_t* row = W + i * K;
        uint16_t s16;
        uint8_t z;
        owq_oracle_search_qparams(row, dense, K, lambda, steps, zsearch, &s16, &z);
        pack_row(row, weak, G, s16, z, qcodes + i * G * 3);
        scales[i] = s16;
        zeros[i] = z;
        for (int32_t c = 0; c < k; c++)
            w_weak[i * k + c] = row[weak_idx[c]];
    }
    free(weak);
    free(dense);
}

void owq_oracle_unpack_codes(const uint32_t* qcodes, int64_t N, int64_t K, uint8_t* codes)
{
    int64_t G = K / 32;
    for (int64_t i = 0; i < N; i++)
        for (int64_t g = 0; g < G; g++)
            for (int c = 0; c < 32; c++)
                codes[i * K + g * 32 + c] = (uint8_t)get_code(qcodes + (i * G + g) * 3, c);
}

/* ---------------------------------------------------------------- linear ---- */

/* The mixed-precision product: the dequantised dense matrix times x plus the
 * fp16 weak columns times the matching activation channels, which the paper's
 * kernel selects on the fly ([PL] "Real-device acceleration", paper
 * "Acceleration on Real Device" p.6; storage as in owq_oracle_pack). Evaluated
 * in fp64 from the packed bytes, one (token, row) pair at a time. */
void owq_oracle_linear_pairs(const uint32_t* qcodes, const uint16_t* scales,
                             const uint8_t* zeros, int64_t N, int64_t K,
                             const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                             const uint16_t* x, int64_t M,
                             const int64_t* pm, const int64_t* pi, int64_t P,
                             double* y, double* bound)
{
    (void)N;
    (void)M;
    int64_t G = K / 32;
    for (int64_t p = 0; p < P; p++) {
        int64_t m = pm[p], i = pi[p];
        double s = owq_oracle_f16_to_f64(scales[i]);
        int z = zeros[i];
        const uint16_t* xm = x + m * K;
        double acc = 0.0, bnd = 0.0;
        for (int64_t j = 0; j < K; j++) {
            int q = get_code(qcodes + (i * G + j / 32) * 3, (int)(j % 32));
            double t = s * (double)(q - z) * owq_oracle_f16_to_f64(xm[j]);
            acc += t;
            bnd += fabs(t);
        }
        for (int32_t c = 0; c < k; c++) {
            double t = owq_oracle_f16_to_f64(w_weak[i * k + c]) *
                       owq_oracle_f16_to_f64(xm[weak_idx[c]]);
            acc += t;
            bnd += fabs(t);
        }
        y[p] = acc;
        bound[p] = bnd;
    }
}

/* The same product for every token and a list of rows, with the rows spread
 * over OpenMP threads (threads <= 0: the OpenMP default). Each output is the
 * sum of the same fp64 terms, in the same order, as owq_oracle_linear_pairs:
 * the row is unpacked once into s (q_j - z) (0 at weak columns), then
 * multiplied by x[m][j] term by term for every token m. y and bound are
 * [M][R]. */
void owq_oracle_linear_rows(const uint32_t* qcodes, const uint16_t* scales,
                            const uint8_t* zeros, int64_t N, int64_t K,
                            const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                            const uint16_t* x, int64_t M,
                            const int64_t* rows, int64_t R, double* y, double* bound,
                            int threads)
{
    (void)N;
    int64_t G = K / 32;
    double* xf = (double*)malloc((size_t)(M * K) * sizeof(double));
    for (int64_t e = 0; e < M * K; e++)
        xf[e] = owq_oracle_f16_to_f64(x[e]);
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
    {
        double* wd = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < R; r++) {
            int64_t i = rows[r];
            double s = owq_oracle_f16_to_f64(scales[i]);
            int z = zeros[i];
            for (int64_t j = 0; j < K; j++)
                wd[j] = s * (double)(get_code(qcodes + (i * G + j / 32) * 3, (int)(j % 32)) - z);
            for (int64_t m = 0; m < M; m++) {
                const double* xm = xf + m * K;
                double acc = 0.0, bnd = 0.0;
                for (int64_t j = 0; j < K; j++) {
                    double t = wd[j] * xm[j];
                    acc += t;
                    bnd += fabs(t);
                }
                for (int32_t c = 0; c < k; c++) {
                    double tw = owq_oracle_f16_to_f64(w_weak[i * k + c]) * xm[weak_idx[c]];
                    acc += tw;
                    bnd += fabs(tw);
                }
                y[m * R + r] = acc;
                bound[m * R + r] = bnd;
            }
        }
        free(wd);
    }
    free(xf);
}

/* ---------------------------------------------------- group-wise scales ---- */

/* Group-wise quantisation on top of OWQ: each output row is split into groups of
 * G consecutive input columns, and every (row, group) gets a step size and zero
 * point of its own ([PL] "Comparison with group-wise quantization", paper p.8,
 * which reports that it adds little on top of OWQ; the group size there is
 * OPTQ's 128). Readings (the pages give no format): G is a multiple of 32 that
 * divides K; each (row, group) is fitted exactly like a row (R1-R4) on the
 * group's dense columns only (R5), so a group of weak columns only, or one whose
 * dense entries are all 0, gets step 1 and zero point 0 (R2); weak columns keep
 * their group's zero point as code; codes keep the R7 layout; scales and zeros
 * are [N][K/G], group-major within a row. */
void owq_oracle_pack_grouped(const uint16_t* W, int64_t N, int64_t K,
                             const int32_t* weak_idx, int32_t k, int64_t G,
                             uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                             uint16_t* w_weak)
{
    uint8_t* weak = (uint8_t*)calloc((size_t)K, 1);
    uint8_t* dense = (uint8_t*)malloc((size_t)K);
    for (int32_t c = 0; c < k; c++)
        weak[weak_idx[c]] = 1;
    for (int64_t j = 0; j < K; j++)
        dense[j] = !weak[j];
    int64_t NG = K / G, CG = G / 32;
    for (int64_t i = 0; i < N; i++) {
        const uint16_t* row = W + i * K;
        for (int64_t g = 0; g < NG; g++) {
            uint16_t s16;
            uint8_t z;
            owq_oracle_qparams(row + g * G, dense + g * G, G, &s16, &z);
            pack_row(row + g * G, weak + g * G, CG, s16, z, qcodes + (i * (K / 32) + g * CG) * 3);
            scales[i * NG + g] = s16;
            zeros[i * NG + g] = z;
        }
        for (int32_t c = 0; c < k; c++)
            w_weak[i * k + c] = row[weak_idx[c]];
    }
    free(weak);
    free(dense);
}

/* The product of the group-wise form for every token and a list of rows (rows
 * over OpenMP threads, threads <= 0: the OpenMP default): y[m][r] = sum_j
 * s_ig (q_ij - z_ig) x[m][j] + sum_c w_weak[i][c] x[m][idx_c] with g = j / G,
 * one fp64 sum per output in column order, then the weak columns; bound[m][r]
 * is the same sum of absolute terms. y and bound are [M][R]. */
void owq_oracle_linear_grouped_rows(const uint32_t* qcodes, const uint16_t* scales,
                                    const uint8_t* zeros, int64_t N, int64_t K, int64_t G,
                                    const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                    const uint16_t* x, int64_t M,
                                    const int64_t* rows, int64_t R, double* y, double* bound,
                                    int threads)
{
    (void)N;
    int64_t NC = K / 32, NG = K / G;
    double* xf = (double*)malloc((size_t)(M * K) * sizeof(double));
    for (int64_t e = 0; e < M * K; e++)
        xf[e] = owq_oracle_f16_to_f64(x[e]);
    int nt = threads > 0 ? threads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
    {
        double* wd = (double*)malloc((size_t)K * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < R; r++) {
            int64_t i = rows[r];
            for (int64_t j = 0; j < K; j++) {
                int64_t g = j / G;
                double s = owq_oracle_f16_to_f64(scales[i * NG + g]);
                int z = zeros[i * NG + g];
                wd[j] = s * (double)(get_code(qcodes + (i * NC + j / 32) * 3, (int)(j % 32)) - z);
            }
            for (int64_t m = 0; m < M; m++) {
                const double* xm = xf + m * K;
                double acc = 0.0, bnd = 0.0;
                for (int64_t j = 0; j < K; j++) {
                    double t = wd[j] * xm[j];
                    acc += t;
                    bnd += fabs(t);
                }
                for (int32_t c = 0; c < k; c++) {
                    double tw = owq_oracle_f16_to_f64(w_weak[i * k + c]) * xm[weak_idx[c]];
                    acc += tw;
                    bnd += fabs(tw);
                }
                y[m * R + r] = acc;
                bound[m * R + r] = bnd;
            }
        }
        free(wd);
    }
    free(xf);
}

/* Effective bit-width. The storage-favoured format drops the zero-filled codes
 * of the k weak columns and adds them in fp16 (16 - 3 = 13 extra bits per weak
 * weight); the latency-favoured format keeps the full 3-bit matrix (16 extra
 * bits per weak weight). Per-row step/zero and the index list are not counted
 * ([PL] "Storage Methods", appendix section 2 pp.10-11). */
double owq_oracle_effective_bits(int64_t K, int64_t k, int latency_favored)
{
    double extra = latency_favored ? 16.0 : 13.0;
    return 3.0 + extra * (double)k / (double)K;
}
