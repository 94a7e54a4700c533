/*
 * owq_oracle.c -- plain, slow CPU oracle of the OWQ hot path.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the package smoke check and the
 * CPU-baseline leg of the benchmark load it; the GPU library never does, and
 * the two share no source. Built with gcc -O2 -ffp-contract=off (no fused
 * multiply-add, no fast-math), so every fp32 step below is one IEEE binary32
 * operation rounded to nearest-even, and every sum is an fp64 sum in loop order.
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
        for (int64_t g = 0; g < G; g++) {
            uint32_t* grp = qcodes + (i * G + g) * 3;
            grp[0] = grp[1] = grp[2] = 0;
            for (int c = 0; c < 32; c++) {
                int64_t j = g * 32 + c;
                int code = weak[j] ? (int)z : owq_oracle_code(row[j], s16, z);
                put_code(grp, c, code);
            }
        }
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
