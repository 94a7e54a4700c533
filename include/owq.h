/*
 * owq.h -- C ABI of libowq.so, the MI355X (gfx950) OWQ hot path.
 *
 * OWQ keeps a few "weak" input columns of each weight matrix in fp16 and
 * quantises the rest to 3 bits. This library computes, entirely in HIP kernels:
 *   calibration  lambda_j = 2 sum_t X[t][j]^2 (Hessian diagonal), the per-column
 *                round-to-nearest error e_j, the column score lambda_j * e_j and the
 *                top-k weak columns;
 *   packing      the latency-favoured format (3-bit codes with weak columns set to
 *                the zero point, per-row fp16 step and uint8 zero, fp16 weak block);
 *   inference    y = x W^T with W given in that format, for any batch M.
 *
 * Pages cited below:
 *   [PL] paperlayer.ai, "OWQ: Outlier-Aware Weight Quantization for Efficient
 *        Fine-Tuning and Inference of Large Language Models" (notes per paper
 *        section; the paper section and page are given in parentheses).
 *   [EL] research.elamur.ai, "OWQ -- paper by Lee et al. (2023) -- summary and ideas".
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked HOST. fp16 data is passed as the
 *     IEEE binary16 bit pattern (uint16_t). All matrices are dense row-major:
 *       W  [N][K]  weights, row i = output channel, column j = input channel
 *       X  [T][K]  calibration activations        x [M][K] layer input
 *       y  [M][N]  layer output
 *   - Packed codes: uint32 [N][K/32][3]. The 32-column group g of row i is the
 *     96-bit little-endian integer qcodes[i][g][0] | qcodes[i][g][1] << 32 |
 *     qcodes[i][g][2] << 64 of 32 three-bit slots, slot s at bits [3s, 3s+3).
 *     Columns 32g + 2p and 32g + 2p + 1 occupy the p-th slot pair: (1,6) (2,7)
 *     (3,8) (4,9) (5,10) (11,16) (12,17) (13,18) (14,19) (15,20) (21,26) (22,27)
 *     (23,28) (24,29) (25,30) (0,31) for p = 0..15. (Only "32 codes per 3 uint32
 *     along K" is fixed by the method; this order lets one 32-bit window of the
 *     group hold both codes of a column pair.)
 *   - The quantiser: per output row, lo = min(0, min w), hi = max(0, max w) over the
 *     fitted columns; step s = fp16_rne((hi - lo) / 7) (IEEE fp32 division), zero
 *     point z = clamp(rint(-lo / s), 0, 7); code(w) = clamp(rint(w / s) + z, 0, 7),
 *     rint = round half to even; dequantised value s * (code - z). A row with
 *     hi == lo, or whose step rounds to fp16 zero, uses s = 1, z = 0. ([PL]
 *     "Low-precision quantization" (paper "Quantization Configuration Search",
 *     pp.4-5): step size, zero point, nearest rounding; [EL] "Key points": min-max
 *     round-to-nearest.)
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Calls
 *     only ENQUEUE work on it; buffers must stay valid until the stream reaches it.
 *   - Arguments are validated synchronously before anything is enqueued; on any
 *     error nothing is enqueued or written and the call returns a non-zero
 *     owq_status (owq_last_error() gives the detail). A HIP launch failure is
 *     reported as OWQ_ERR_HIP.
 *   - Ownership: the caller allocates and owns every buffer; the library keeps no
 *     pointer after a call returns and allocates no device memory in these calls.
 *   - Thread safety: no mutable global state except the thread-local error text.
 *   - Limits: 1 <= N, M, T; 32 <= K <= 65536 with K % 32 == 0; 0 <= k <= K;
 *     bits == 3. Device pointers must be aligned to their element size, qcodes and
 *     x / X / W to 16 bytes. Inputs must be finite.
 */
#ifndef OWQ_H
#define OWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    OWQ_OK = 0,
    OWQ_ERR_NULL = 1,        /* a required pointer is NULL */
    OWQ_ERR_SHAPE = 2,       /* N, K, M or T out of range, or K % 32 != 0 */
    OWQ_ERR_RANGE = 3,       /* k outside [0, K] */
    OWQ_ERR_ALIGN = 4,       /* a device pointer is misaligned */
    OWQ_ERR_UNSUPPORTED = 5, /* bits != 3, or a batched call mixes unsupported shapes */
    OWQ_ERR_WORKSPACE = 6,   /* workspace smaller than owq_calibrate_workspace_bytes */
    OWQ_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed */
} owq_status;

/* Static text for a status code; never NULL. */
const char* owq_status_string(owq_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* owq_last_error(void);

/* ------------------------------------------------------------- calibration --- */

/* Bytes of device workspace owq_calibrate_score needs for these sizes
 * (0 for invalid sizes). */
size_t owq_calibrate_workspace_bytes(int64_t N, int64_t K, int64_t T);

/* Column sensitivity of one linear layer.
 *   lambda[j] = 2 * sum_t X[t][j]^2                       (fp64, [K])
 *   score[j]  = lambda[j] * sum_i (W[i][j] - deq_i(code_i(W[i][j])))^2  (fp64, [K])
 * where (s_i, z_i) fit row i over ALL K columns.
 * The layer-wise error ||W X^T - W^ X^T||^2 splits into per-output-row quadratic
 * errors sharing the Hessian 2 X^T X, whose diagonal is lambda ([PL] "Error
 * Decomposition", "Error Analysis" (paper p.3; appendix section 1, p.10)); the
 * sensitivity of a column is its squared perturbation norm times its Hessian
 * diagonal element ([PL] "Weak-column selection" (paper p.4)).
 * W: fp16 [N][K]; X: fp16 [T][K]; lambda, score: fp64 [K] (outputs; may not alias).
 * workspace: device scratch of >= owq_calibrate_workspace_bytes(N, K, T) bytes,
 * 256-byte aligned; its contents on entry are ignored. Two calls may share a
 * workspace only if they are ordered (e.g. on one stream).
 * Results are bitwise deterministic for given inputs. */
owq_status owq_calibrate_score(const uint16_t* W, int64_t N, int64_t K,
                               const uint16_t* X, int64_t T,
                               double* lambda, double* score,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Weak-column selection: the k columns of largest score (ties: the lower column
 * index wins), written to weak_idx[0..k) in strictly ascending order ([PL]
 * "Weak-column selection" (paper p.4): the top-k columns by sensitivity are kept
 * in fp16). score: fp64 [K] (any finite values); weak_idx: int32 [k] (output;
 * may be NULL iff k == 0). k == 0 enqueues nothing. */
owq_status owq_select_weak(const double* score, int64_t K, int32_t k,
                           int32_t* weak_idx, void* stream);

/* ------------------------------------------------------------------- pack --- */

/* Latency-favoured OWQ storage of one layer ([PL] "Storage Methods" (paper
 * appendix section 2, pp.10-11): the complete low-precision matrix with the weak
 * columns zero-filled, plus the weak columns in fp16). Each row is fitted on its
 * dense (non-weak) columns only; weak columns are excluded from quantisation
 * ([PL] "Weak-column selection" (paper p.4)); their codes are the zero point, so
 * they dequantise to 0.
 * W: fp16 [N][K]. weak_idx: int32 [k], strictly ascending in [0, K) (NULL iff
 * k == 0; the order is the caller's contract and is not re-checked on the GPU).
 * Outputs: qcodes uint32 [N][K/32][3]; scales fp16 [N]; zeros uint8 [N] (0..7);
 * w_weak fp16 [N][k] with w_weak[i][c] = W[i][weak_idx[c]] (NULL iff k == 0).
 * Bitwise identical to the reference definition above. */
owq_status owq_pack(const uint16_t* W, int64_t N, int64_t K,
                    const int32_t* weak_idx, int32_t k,
                    uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                    uint16_t* w_weak, void* stream);

/* ----------------------------------------------------------------- linear --- */

/* One packed layer, as produced by owq_pack. The struct itself is HOST memory;
 * its pointers are device pointers. */
typedef struct {
    int64_t N, K;               /* output rows, input columns */
    int32_t k;                  /* weak columns */
    int32_t bits;               /* must be 3 */
    const uint32_t* qcodes;     /* [N][K/32][3] */
    const uint16_t* scales;     /* fp16 [N] */
    const uint8_t* zeros;       /* [N] */
    const int32_t* weak_idx;    /* [k], ascending (NULL iff k == 0) */
    const uint16_t* w_weak;     /* fp16 [N][k] (NULL iff k == 0) */
} owq_layer;

/* Mixed-precision product of the 3-bit dense matrix and the fp16 weak columns
 * ([PL] "Real-device acceleration" (paper "Acceleration on Real Device", p.6): a
 * 3-bit x fp16 kernel that picks the weak-column activation channels on the fly):
 *   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][weak_idx[c]]
 * computed with fp32 accumulation and rounded to fp16 (nearest-even).
 * L: HOST pointer to the layer; x: fp16 [M][K]; y: fp16 [M][N] (output, must not
 * alias x or the layer). M <= 2 runs an HBM-streaming kernel on the vector ALUs,
 * 3 <= M <= 16 a streaming kernel that multiplies on the matrix cores, larger M a
 * tiled matrix-core (MFMA) GEMM; all compute the same definition. The environment
 * variable OWQ_DECODE (read at each call) overrides the first split: "matrix"
 * sends every M <= 16 to the matrix-core streaming kernel, "vector" keeps M <= 4
 * on the vector ALUs; OWQ_GEMM_MIN_M (read once) moves the GEMM bound. */
owq_status owq_linear(const owq_layer* L, const uint16_t* x, int64_t M,
                      uint16_t* y, void* stream);

/* `count` independent linears with the same M in ONE kernel launch per 16 layers,
 * with the results owq_linear's decode kernels would give one by one (the layers
 * run in order of decreasing K inside the launch). Ls: HOST array [count] of
 * layers; xs, ys: HOST arrays [count] of device pointers with the shapes
 * owq_linear expects. Returns OWQ_ERR_UNSUPPORTED unless 1 <= M <= 16 and
 * 1 <= count <= 64. */
owq_status owq_linear_batched(const owq_layer* Ls, const uint16_t* const* xs,
                              uint16_t* const* ys, int32_t count, int64_t M,
                              void* stream);

/* ------------------------------------------------- measurement reference --- */

/* Not a step of the method: a read-only HBM stream with the M = 1 decode
 * kernel's geometry (wavefronts of 6 x 768 contiguous bytes, 12 bytes per lane
 * per load), for reading the decode rate against a measured ceiling.
 * src: device buffer of `bytes` bytes (12 <= bytes <= 2^40, bytes % 12 == 0,
 * 4-byte aligned). sink: device uint32 [sink_words] (output), sink_words >=
 * owq_stream_read_sink_words(bytes); word w receives the XOR of the 32-bit words
 * of bytes [4608 w, 4608 (w + 1)) of src (the last one zero-padded). Returns
 * OWQ_ERR_NULL, OWQ_ERR_SHAPE, OWQ_ERR_ALIGN or OWQ_ERR_RANGE (sink too short)
 * before any launch. */
int64_t owq_stream_read_sink_words(int64_t bytes);
owq_status owq_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                           int64_t sink_words, void* stream);

#ifdef __cplusplus
}
#endif
#endif
