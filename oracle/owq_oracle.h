/*
 * owq_oracle.h -- plain CPU oracle of the OWQ hot path (TEST INFRASTRUCTURE).
 *
 * Only the test-suite, the package smoke check and the CPU-baseline leg of the
 * benchmark may load this library. The GPU library shares no code with it.
 *
 * Pages cited in this file and in owq_oracle.c:
 *   [PL] paperlayer.ai, "OWQ: Outlier-Aware Weight Quantization for Efficient
 *        Fine-Tuning and Inference of Large Language Models" (per-section notes;
 *        each cited heading names the paper section and page it summarises).
 *   [EL] research.elamur.ai, "OWQ -- paper by Lee et al. (2023) -- summary and ideas".
 *
 * Data conventions: fp16 values are IEEE binary16 bit patterns (uint16_t).
 * W is [N][K] row-major (row i = output channel, column j = input channel).
 * X is [T][K] calibration activations, x is [M][K] layer input, y is [M][N].
 * Packed codes: uint32 [N][K/32][3]; a 32-column group is the 96-bit little-endian
 * integer w0 | w1<<32 | w2<<64 of 32 three-bit slots (slot s at bits [3s, 3s+3)),
 * and columns 2p, 2p+1 of the group occupy the p-th slot pair (1,6) (2,7) (3,8)
 * (4,9) (5,10) (11,16) (12,17) (13,18) (14,19) (15,20) (21,26) (22,27) (23,28)
 * (24,29) (25,30) (0,31).
 */
#ifndef OWQ_ORACLE_H
#define OWQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* IEEE binary16 -> binary64, exact. */
double owq_oracle_f16_to_f64(uint16_t h);
/* IEEE binary32 -> binary16, round to nearest, ties to even. */
uint16_t owq_oracle_f32_to_f16(float f);

/* Min-max step size and zero point of one row over the columns with use[j] != 0
 * (use == NULL: every column). Writes the fp16 step bits and the zero point. */
void owq_oracle_qparams(const uint16_t* row, const uint8_t* use, int64_t K,
                        uint16_t* s16, uint8_t* z);
/* Round-to-nearest 3-bit code of one weight under (s16, z). */
int owq_oracle_code(uint16_t w, uint16_t s16, uint8_t z);

/* lambda[j] = 2 * sum_t X[t][j]^2 (Hessian diagonal), fp64. */
void owq_oracle_hessian_diag(const uint16_t* X, int64_t T, int64_t K, double* lambda);
/* e[j] = sum_i (W[i][j] - deq(code(W[i][j])))^2 under each row's full-row fit. */
void owq_oracle_rtn_col_err(const uint16_t* W, int64_t N, int64_t K, double* e);
/* lambda and score[j] = lambda[j] * e[j]. */
void owq_oracle_calibrate_score(const uint16_t* W, int64_t N, int64_t K,
                                const uint16_t* X, int64_t T,
                                double* lambda, double* score);
/* The k columns of largest score (ties: lower index first), written ascending. */
void owq_oracle_select_weak(const double* score, int64_t K, int32_t k, int32_t* weak_idx);

/* Latency-favoured pack: dense codes with weak columns set to the zero point,
 * per-row fp16 step and uint8 zero, and the fp16 weak columns [N][k]. */
void owq_oracle_pack(const uint16_t* W, int64_t N, int64_t K,
                     const int32_t* weak_idx, int32_t k,
                     uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                     uint16_t* w_weak);
/* Inverse of the bit layout: codes [N][K] (values 0..7). */
/* Truncation-aware (step, zero point) of one row: a 2D grid search minimising
 * the row's (optionally lambda-weighted) squared reconstruction error over the
 * columns with use[j] != 0; grid and tie rule in owq_oracle.c (readings S1-S4).
 * steps = number of step factors 1 - a/40; zsearch = 0 keeps the min-max zero
 * point of each step. */
void owq_oracle_search_qparams(const uint16_t* row, const uint8_t* use, int64_t K,
                               const double* lambda, int steps, int zsearch,
                               uint16_t* s16, uint8_t* z);
/* Latency-favoured pack with searched per-row parameters (OpenMP over rows). */
void owq_oracle_pack_search(const uint16_t* W, int64_t N, int64_t K,
                            const int32_t* weak_idx, int32_t k, const double* lambda,
                            int steps, int zsearch,
                            uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                            uint16_t* w_weak, int threads);
/* Storage-favoured form: only the dense columns' codes, ascending, 32 per group
 * (last group filled with the zero point): qcodes [N][ceil((K-k)/32)][3]; the
 * steps, zero points and weak block are the latency-favoured pack's. */
void owq_oracle_pack_storage(const uint16_t* W, int64_t N, int64_t K,
                             const int32_t* weak_idx, int32_t k,
                             uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                             uint16_t* w_weak);
/* Its product for every token of the listed rows (OpenMP over rows); x is the
 * full [M][K] input. y, bound: [M][R]. */
void owq_oracle_linear_storage_rows(const uint32_t* qcodes, const uint16_t* scales,
                                    const uint8_t* zeros, int64_t N, int64_t K,
                                    const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                    const uint16_t* x, int64_t M,
                                    const int64_t* rows, int64_t R, double* y, double* bound,
                                    int threads);
/* Backward of the mixed-precision linear for weak-column tuning: dx = dy W
 * ([M][K]) and dw_weak = dy^T x[:, idx] ([N][k]), fp64, with bounds (sums of
 * |terms|); either output pair may be NULL. OpenMP over columns / rows. */
void owq_oracle_linear_backward(const uint32_t* qcodes, const uint16_t* scales,
                                const uint8_t* zeros, int64_t N, int64_t K,
                                const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                const uint16_t* x, const uint16_t* dy, int64_t M,
                                double* dx, double* dx_bound, double* dw, double* dw_bound,
                                int threads);
/* IEEE binary64 -> binary16, round to nearest, ties to even. */
uint16_t owq_oracle_f64_to_f16(double f);
/* OPTQ with the weak columns last: U [K][K] (upper; H^-1 = U^T U for the damped
 * Hessian 2 X^T X in the order dense-then-weak), readings P1-P3 in owq_oracle.c. */
void owq_oracle_optq_factor(const uint16_t* X, int64_t T, int64_t K, const int32_t* weak_idx, int32_t k,
                            double* U, int threads);
/* The sequential quantisation of every row with compensation through U
 * (readings P4-P6), latency-favoured outputs. */
void owq_oracle_optq_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* weak_idx, int32_t k,
                          const double* U, uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                          uint16_t* w_weak, int threads);
void owq_oracle_unpack_codes(const uint32_t* qcodes, int64_t N, int64_t K, uint8_t* codes);

/* y and the error bound for P (token m, row i) pairs, from the packed layer.
 * y[p]     = sum_j s_i (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
 * bound[p] = sum_j |s_i (q_ij - z_i) x[m][j]| + sum_c |w_weak[i][c] x[m][idx_c]| */
void owq_oracle_linear_pairs(const uint32_t* qcodes, const uint16_t* scales,
                             const uint8_t* zeros, int64_t N, int64_t K,
                             const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                             const uint16_t* x, int64_t M,
                             const int64_t* pm, const int64_t* pi, int64_t P,
                             double* y, double* bound);

/* All M tokens of the listed rows (OpenMP over rows; threads <= 0: default).
 * Each output equals owq_oracle_linear_pairs' for that (token, row) bit for bit.
 * y[m][r], bound[m][r] for row rows[r]. */
/* Group-wise scales on top of OWQ: a step and zero point per (row, group of G
 * columns), G a multiple of 32 dividing K; scales and zeros are [N][K/G]. */
void owq_oracle_pack_grouped(const uint16_t* W, int64_t N, int64_t K,
                             const int32_t* weak_idx, int32_t k, int64_t G,
                             uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                             uint16_t* w_weak);
void owq_oracle_linear_grouped_rows(const uint32_t* qcodes, const uint16_t* scales,
                                    const uint8_t* zeros, int64_t N, int64_t K, int64_t G,
                                    const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                                    const uint16_t* x, int64_t M,
                                    const int64_t* rows, int64_t R, double* y, double* bound,
                                    int threads);
void owq_oracle_linear_rows(const uint32_t* qcodes, const uint16_t* scales,
                            const uint8_t* zeros, int64_t N, int64_t K,
                            const int32_t* weak_idx, const uint16_t* w_weak, int32_t k,
                            const uint16_t* x, int64_t M,
                            const int64_t* rows, int64_t R, double* y, double* bound,
                            int threads);

/* Effective bits per weight: 3 + 13k/K (storage-favoured) or 3 + 16k/K
 * (latency-favoured, zero-filled dense matrix kept). */
double owq_oracle_effective_bits(int64_t K, int64_t k, int latency_favored);

#ifdef __cplusplus
}
#endif
#endif
