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
 *   - Thread safety: no mutable global state except the thread-local error text
 *     and, for owq_calibrate_score_noalloc, the per-device address of its static
 *     scratch array (looked up once per device, under a lock).
 *   - Limits: 1 <= N, M, T; 32 <= K <= 65536 with K % 32 == 0; 0 <= k <= K;
 *     bits == 3. Device pointers must be aligned to their element size (qcodes and
 *     weak_idx: 4 bytes, fp16 arrays: 2 bytes, fp64 arrays: 8 bytes), and x / X / W
 *     to 16 bytes (they are read in 16-byte pieces). Inputs must be finite.
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

/* owq_calibrate_score for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * buffer the library itself holds on each GPU (a static device array of
 * owq_calibrate_noalloc_max_workspace() bytes, created when the library is
 * loaded on that GPU and kept until the process ends; its address is looked up
 * once per device, on the first call with that device current). The call
 * makes no allocation. It runs on the CURRENT device, and `stream` must belong
 * to it. Returns OWQ_ERR_WORKSPACE, before any launch, when
 * owq_calibrate_workspace_bytes(N, K, T) exceeds that maximum. Every call on a
 * GPU shares that GPU's buffer: calls that overlap on one GPU (on different
 * streams, or from different threads) race and give undefined results; calls
 * ordered on one stream are safe. The buffer's contents from a previous call
 * are never read. Other arguments and errors as owq_calibrate_score. */
owq_status owq_calibrate_score_noalloc(const uint16_t* W, int64_t N, int64_t K,
                                       const uint16_t* X, int64_t T,
                                       double* lambda, double* score, void* stream);
/* Bytes of the library-held workspace owq_calibrate_score_noalloc uses. */
size_t owq_calibrate_noalloc_max_workspace(void);

/* One linear of owq_calibrate_score_batched: its arguments as
 * owq_calibrate_score's (device pointers; lambda and score are outputs). */
typedef struct owq_calib_item {
    const uint16_t* W;  /* fp16 [N][K] */
    int64_t N, K;
    const uint16_t* X;  /* fp16 [T][K] */
    int64_t T;
    double* lambda;     /* fp64 [K] */
    double* score;      /* fp64 [K] */
} owq_calib_item;

/* Bytes of device workspace owq_calibrate_score_batched needs for these
 * items: their owq_calibrate_workspace_bytes, each rounded up to 256 bytes (0
 * for invalid sizes or count outside 1..64). */
size_t owq_calibrate_batched_workspace_bytes(const owq_calib_item* items, int32_t count);

/* owq_calibrate_score for `count` linears (e.g. the 7 of a decoder layer), bit
 * for bit the same results, in count + 2 kernel launches instead of 3 per
 * linear: launch s holds the first pass of linear s (X column sums, W row
 * fits), the error pass of linear s - 1 (which re-reads a W the previous launch
 * just streamed) and the final pass of linear s - 2 ([PL] "Weak-column
 * selection" (paper p.4), as owq_calibrate_score). items: HOST array [count].
 * workspace: >= owq_calibrate_batched_workspace_bytes(items, count) bytes,
 * 256-byte aligned; item l's part starts at the sum of the earlier items'
 * rounded sizes. Returns OWQ_ERR_UNSUPPORTED unless 1 <= count <= 64; other
 * errors as owq_calibrate_score, reported with the item's index. */
owq_status owq_calibrate_score_batched(const owq_calib_item* items, int32_t count, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Weak-column selection: the k columns of largest score (ties: the lower column
 * index wins), written to weak_idx[0..k) in strictly ascending order ([PL]
 * "Weak-column selection" (paper p.4): the top-k columns by sensitivity are kept
 * in fp16). score: fp64 [K] (any finite values); weak_idx: int32 [k] (output;
 * may be NULL iff k == 0). k == 0 enqueues nothing. */
owq_status owq_select_weak(const double* score, int64_t K, int32_t k,
                           int32_t* weak_idx, void* stream);

/* `count` independent weak-column selections (e.g. the 7 linears of a decoder
 * layer) with the results owq_select_weak would give one by one, in one kernel
 * launch (with the widest block shape any of them needs; selections with
 * K > 16384 get one launch each): every selection is a latency-bound single
 * workgroup, so they run side by side.
 * scores, weak_idxs: HOST arrays [count] of device pointers; Ks, ks: HOST arrays
 * [count]; each selection's arguments as owq_select_weak's. Returns
 * OWQ_ERR_UNSUPPORTED unless 1 <= count <= 64; other errors as owq_select_weak,
 * reported with the selection's index. */
owq_status owq_select_weak_batched(const double* const* scores, const int64_t* Ks, const int32_t* ks,
                                   int32_t* const* weak_idxs, int32_t count, void* stream);

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

/* One linear of owq_pack_batched: owq_pack's arguments (device pointers). */
typedef struct owq_pack_item {
    const uint16_t* W;        /* fp16 [N][K] */
    int64_t N, K;
    const int32_t* weak_idx;  /* int32 [k], ascending (may be NULL iff k == 0) */
    int32_t k;
    uint32_t* qcodes;         /* [N][K/32][3] (output) */
    uint16_t* scales;         /* fp16 [N] (output) */
    uint8_t* zeros;           /* uint8 [N] (output) */
    uint16_t* w_weak;         /* fp16 [N][k] (output; may be NULL iff k == 0) */
} owq_pack_item;

/* owq_pack for `count` linears (e.g. the 7 of a decoder layer), bit for bit the
 * same outputs ([PL] "Storage Methods", paper appendix section 2, as owq_pack),
 * with the linears of one kernel form in one launch (every row is independent,
 * so the rows of all of them stream side by side). items: HOST array [count].
 * Returns OWQ_ERR_UNSUPPORTED unless 1 <= count <= 64; other errors as
 * owq_pack, reported with the item's index. */
owq_status owq_pack_batched(const owq_pack_item* items, int32_t count, void* stream);

/* owq_pack with each row's step size and zero point chosen by a truncation-aware
 * 2D grid search over both, before the codes are formed ([PL] "Low-precision
 * quantization" (paper "Quantization Configuration Search", pp.4-5): a grid
 * search over step size and zero point with nearest rounding and truncation, to
 * narrow the range and reduce the reconstruction error; effect on quality: [PL]
 * "Quantization quality", p.5). Per row, over its dense columns only:
 *   grid    steps s_a = fp16_rne(s_mm * (1 - a/40)), a = 0..31, where s_mm =
 *           (hi - lo) / 7 is the fp32 min-max step of the quantiser above (a = 0
 *           is the min-max step; a step that rounds to fp16 zero is skipped),
 *           times zero points z = 0..7;
 *   error   E(a, z) = sum_j omega_j (w_j - s_a (code_j - z))^2 over the dense
 *           columns in ascending order, code_j = clamp(rint(w_j / s_a) + z, 0, 7),
 *           omega_j = lambda[j] if lambda is non-NULL, else 1, each term
 *           (d * d) then times omega_j, summed in fp64;
 *   choice  the smallest E; ties go to the smaller a, then the smaller z.
 * A degenerate row (hi == lo, or s_mm rounding to fp16 zero) keeps s = 1, z = 0.
 * Weights outside the chosen range are truncated to the nearest end code. The
 * format, weak columns and outputs are owq_pack's; owq_linear reads it unchanged.
 * lambda: fp64 [K] (e.g. owq_calibrate_score's Hessian diagonal, so that E is
 * the row's output error under the diagonal Hessian) or NULL (plain squared
 * weight error). Other arguments and errors as owq_pack. The codes, steps and
 * zero points are bitwise identical to that definition. */
owq_status owq_pack_search(const uint16_t* W, int64_t N, int64_t K,
                           const int32_t* weak_idx, int32_t k, const double* lambda,
                           uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                           uint16_t* w_weak, void* stream);

/* The storage-favoured OWQ form ([PL] "Storage Methods" (paper appendix section
 * 2, pp.10-11): the zero-filled weak columns are removed from the low-precision
 * matrix, which saves their 3 bits per weight (3 + 13k/K bits instead of
 * 3 + 16k/K) at the price of extra work in the product). Row i keeps the codes of
 * its dense columns only, in ascending column order, 32 to a group in the slot
 * layout above; the last group of a row is filled with the zero point (it
 * dequantises to 0). qcodes: uint32 [N][ceil((K - k)/32)][3] (may be NULL when
 * k == K: no codes). Steps, zero points and the weak block are owq_pack's (each
 * row fitted on its dense columns); other arguments and errors as owq_pack. The
 * codes are bitwise identical to owq_pack's with the weak columns dropped. */
owq_status owq_pack_storage(const uint16_t* W, int64_t N, int64_t K,
                            const int32_t* weak_idx, int32_t k,
                            uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                            uint16_t* w_weak, void* stream);

/* Bytes of device workspace owq_pack_optq needs (0 for invalid sizes): two
 * K x K fp64 matrices (the Hessian, factored in place, and the inverse factor),
 * an N x K fp64 working copy of W and N x K bytes of codes. */
size_t owq_pack_optq_workspace_bytes(int64_t N, int64_t K, int32_t k);

/* Latency-favoured pack (owq_pack's outputs and format) with the dense columns
 * quantised by OPTQ's sequential column-by-column quantisation and error
 * compensation, the weak columns moved to the end so that their fp16 values
 * absorb compensation without being quantised, on the Hessian 2 X^T X that the
 * weak-column selection shares ([PL] "OPTQ: Weight Quantization for LLMs"
 * (pp.2-3), "OWQ: Outlier-aware Weight Quantization" (p.4), "Quantization
 * efficiency" (paper "Quantization Speed", p.7), "B Experiment Details" (p.10)).
 * Definition (the pages give the method; these details are the library's):
 *   H = 2 X^T X in fp64; a zero diagonal entry is set to 1, then every diagonal
 *   entry gains 0.01 times the mean diagonal; the columns are ordered dense
 *   ascending then weak ascending; U is the upper-triangular factor with H^-1 =
 *   U^T U (the inverse of the Cholesky factor of H taken in reversed order);
 *   each row's step and zero point are owq_pack's (min-max over its dense
 *   columns); in that order, column a of a row gets the code clamp(rint(w_a /
 *   s) + z, 0, 7) of its current (compensated, fp64) weight, and its error
 *   e = (w_a - s (q - z)) / U_aa is subtracted from every later column b as
 *   e U_ab, in batches of 128 columns (within a batch column by column; each
 *   later batch receives the batch's sum over a of e_a U_ab in column order);
 *   w_weak is the compensated weak weights rounded to fp16 (nearest-even); weak
 *   codes are the zero point.
 * X: fp16 [T][K] calibration input; other arguments and outputs as owq_pack.
 * workspace: >= owq_pack_optq_workspace_bytes(N, K, k) bytes, 256-byte aligned.
 * Every sum runs in the definition's order, so the outputs are bitwise
 * reproducible. An offline step: the Cholesky factor takes one launch per
 * column. */
owq_status owq_pack_optq(const uint16_t* W, int64_t N, int64_t K,
                         const uint16_t* X, int64_t T,
                         const int32_t* weak_idx, int32_t k,
                         uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                         uint16_t* w_weak, void* workspace, size_t workspace_bytes,
                         void* stream);

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
 * alias x or the layer). M <= 2 runs an HBM-streaming kernel that decodes on the
 * vector ALUs (one token multiplies there too, two on the matrix cores;
 * OWQ_GEMV_PRODUCTS=dot2|mfma, read at each call, overrides that choice),
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

/* Bytes of device workspace owq_linear_storage needs (0 for invalid sizes). */
size_t owq_linear_storage_workspace_bytes(int64_t K, int32_t k, int64_t M);

/* owq_linear on a layer in the storage-favoured form (owq_pack_storage): the same
 * product, y[m][i] = s_i sum_{dense j} (q_ij - z_i) x[m][j] + sum_c w_weak[i][c]
 * x[m][weak_idx[c]], fp32 accumulation, fp16 output. L->K is the full column
 * count and L->qcodes the storage-form codes (NULL allowed when k == K). The
 * extra work of this form: x at the dense columns is gathered into the
 * workspace, the dense product runs as a layer of ceil((K-k)/32)*32 columns, and
 * the weak columns' product goes into the same fp32 sum when that product runs
 * on the vector-ALU decode (M <= 2 by default; one fp16 rounding), else it is
 * added to y afterwards (y then rounded to fp16 twice when 0 < k < K). workspace: >= owq_linear_storage_workspace_bytes(K, k,
 * M) bytes, 256-byte aligned, contents ignored; calls sharing it must be ordered.
 * Errors as owq_linear, plus OWQ_ERR_WORKSPACE. */
owq_status owq_linear_storage(const owq_layer* L, const uint16_t* x, int64_t M,
                              uint16_t* y, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------- group-wise form --- */

/* Group-wise scales on top of OWQ ([PL] "Comparison with group-wise
 * quantization", paper p.8: a step size and zero point per group of input
 * columns, which the pages find adds little to OWQ; their grouped baseline uses
 * groups of 128). Definition (the pages give no format; these details are the
 * library's): row i is split into groups of G consecutive columns; each (row,
 * group) is fitted like a row of owq_pack on the group's dense columns only
 * (lo = min(0, min w), hi = max(0, max w), step fp16((hi - lo) / 7), zero point
 * clamp(rint(-lo / step), 0, 7); hi == lo, or a step that rounds to fp16 zero,
 * gives step 1 and zero point 0, as for a group of weak columns only); dense
 * codes are clamp(rint(w / step) + z, 0, 7), weak columns take their group's
 * zero point; codes in owq_pack's slot layout. G must be a power of two from 32
 * to 2048 dividing K (OWQ_ERR_UNSUPPORTED otherwise).
 * scales: fp16 [N][K/G], zeros: uint8 [N][K/G] (group-major within a row);
 * other arguments, layouts and errors as owq_pack. Bitwise reproducible. */
owq_status owq_pack_grouped(const uint16_t* W, int64_t N, int64_t K,
                            const int32_t* weak_idx, int32_t k, int64_t G,
                            uint32_t* qcodes, uint16_t* scales, uint8_t* zeros,
                            uint16_t* w_weak, void* stream);

/* One layer in the group-wise form (owq_pack_grouped). HOST struct, device
 * pointers. */
typedef struct {
    int64_t N, K, G;            /* output rows, input columns, columns per group */
    int32_t k;                  /* weak columns */
    int32_t bits;               /* must be 3 */
    const uint32_t* qcodes;     /* [N][K/32][3] */
    const uint16_t* scales;     /* fp16 [N][K/G] */
    const uint8_t* zeros;       /* [N][K/G] */
    const int32_t* weak_idx;    /* [k], ascending (NULL iff k == 0) */
    const uint16_t* w_weak;     /* fp16 [N][k] (NULL iff k == 0) */
} owq_grouped_layer;

/* Product of the group-wise form ([PL] "Comparison with group-wise
 * quantization", p.8, on the product of "Real-device acceleration", p.6):
 *   y[m][i] = sum_g s_ig sum_{j in g} (q_ij - z_ig) x[m][j] + sum_c w_weak[i][c] x[m][weak_idx[c]]
 * with exact fp16 products, fp32 sums (one per 32 columns, scaled by its
 * group's step) and an fp16 output (nearest-even). x: fp16 [M][K], y: fp16
 * [M][N] (must not alias x or the layer). One launch of the vector-ALU decode
 * kernel (owq_linear's, in its group-wise mode) per 4 tokens. Errors as
 * owq_linear, plus OWQ_ERR_UNSUPPORTED for a G that owq_pack_grouped rejects. */
owq_status owq_linear_grouped(const owq_grouped_layer* L, const uint16_t* x, int64_t M,
                              uint16_t* y, void* stream);

/* `count` independent group-wise linears with the same M (e.g. the 7 linears of
 * a decoder layer) in ONE decode launch per 16 layers, bit for bit the results of
 * owq_linear_grouped one by one. Ls: HOST array [count]; xs, ys: HOST arrays
 * [count] of device pointers with owq_linear_grouped's shapes. Returns
 * OWQ_ERR_UNSUPPORTED unless 1 <= M <= 4 and 1 <= count <= 64. */
owq_status owq_linear_grouped_batched(const owq_grouped_layer* Ls, const uint16_t* const* xs,
                                      uint16_t* const* ys, int32_t count, int64_t M, void* stream);

/* Bytes of device workspace owq_linear_storage_batched needs for these layers
 * at M tokens: their owq_linear_storage_workspace_bytes, each rounded up to 256
 * bytes (0 for invalid sizes or count outside 1..64). */
size_t owq_linear_storage_batched_workspace_bytes(const owq_layer* Ls, int32_t count, int64_t M);

/* owq_linear_storage for `count` layers at the same M (e.g. the 7 linears of a
 * decoder layer), bit for bit the same outputs ([PL] "Storage Methods", paper
 * appendix section 2, as owq_linear_storage), in three launches instead of three
 * per layer: the dense-column gathers of every layer, the dense products (one
 * decode launch when M is in its range), the weak columns of every layer. Ls,
 * xs, ys: HOST arrays [count] (structs and device pointers). workspace: >=
 * owq_linear_storage_batched_workspace_bytes(Ls, count, M) bytes, 256-byte
 * aligned; layer l's part starts at the sum of the earlier layers' rounded
 * sizes. Returns OWQ_ERR_UNSUPPORTED unless 1 <= count <= 64; other errors as
 * owq_linear_storage, reported with the layer's index. */
owq_status owq_linear_storage_batched(const owq_layer* Ls, const uint16_t* const* xs, uint16_t* const* ys,
                                      int32_t count, int64_t M, void* workspace, size_t workspace_bytes,
                                      void* stream);

/* ------------------------------------------ backward (weak-column tuning) --- */

/* Bytes of device workspace owq_linear_backward needs to produce dx (0 for
 * invalid sizes). */
size_t owq_linear_backward_workspace_bytes(int64_t N, int64_t K, int32_t k);

/* Backward of owq_linear for Weak Column Tuning, which trains only the fp16 weak
 * columns and keeps the 3-bit dense matrix frozen ([PL] "Weak Column Tuning"
 * (paper "PEFT with Weak Column Tuning", p.5); the trainable block is w_weak,
 * N x k: "Learnable Parameters" (appendix section 3, p.13)). With W the
 * dequantised dense matrix (0 at the weak columns) plus the weak columns and the
 * upstream gradient dy = dL/dy:
 *   dx[m][j]      = sum_i dy[m][i] W[i][j]         fp32 sums, fp16 [M][K]
 *   dw_weak[i][c] = sum_m dy[m][i] x[m][idx_c]     fp32 sums, fp32 [N][k]
 * L: HOST pointer to the packed layer (latency-favoured form); x: fp16 [M][K]
 * (the layer input; read only for dw_weak, may be NULL otherwise); dy: fp16
 * [M][N]; dx (may be NULL) and dw_weak (may be NULL) are outputs. dx is the
 * transposed 3-bit product, summed over row slices in a fixed order (bitwise
 * deterministic): up to 4 tokens on the vector ALUs (exact products), more on
 * the matrix cores 16 tokens per pass (exact products: dy times s (q - z) split
 * into two fp16 values; fp32 products for a 512-row slice holding a step above
 * 9352; the environment variable OWQ_BACKWARD=vector, read at each call, keeps
 * the vector form). workspace: >=
 * owq_linear_backward_workspace_bytes(N, K, k) bytes, 256-byte aligned, needed
 * only for dx. Errors as owq_linear, plus OWQ_ERR_WORKSPACE. */
owq_status owq_linear_backward(const owq_layer* L, const uint16_t* x, const uint16_t* dy,
                               int64_t M, uint16_t* dx, float* dw_weak,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace owq_linear_backward_batched needs for dx of the
 * `count` layers Ls (HOST array): the layers' own sizes, each rounded up to 256
 * bytes (0 for invalid sizes or count outside 1..64). */
size_t owq_linear_backward_batched_workspace_bytes(const owq_layer* Ls, int32_t count);

/* owq_linear_backward for `count` layers at once (the linears of one decoder
 * layer in the same backward step, e.g. q/k/v or gate/up, which read one input):
 * the same definition and the same results, bit for bit, as one call per layer,
 * with the layers' work in ONE kernel launch (plus one for the final sums) per 16
 * layers and 4 tokens instead of two per layer ([PL] "Weak Column Tuning" (paper
 * "PEFT with Weak Column Tuning", p.5)). Ls: HOST array [count] of layers; xs,
 * dys, dxs, dws: HOST arrays [count] of device pointers with the meanings and
 * shapes of owq_linear_backward's x, dy, dx, dw_weak (xs, dxs, dws may be NULL,
 * or hold NULL entries, for "not needed" / "not wanted"), all with the same M.
 * workspace: >= owq_linear_backward_batched_workspace_bytes over the layers
 * that want dx (the full Ls is always enough), 256-byte aligned; layer l's part
 * starts at the sum of the rounded sizes of the earlier layers that want dx.
 * Returns OWQ_ERR_UNSUPPORTED unless 1 <= count <= 64; other errors as
 * owq_linear_backward, reported with the layer's index. */
owq_status owq_linear_backward_batched(const owq_layer* Ls, const uint16_t* const* xs,
                                       const uint16_t* const* dys, int32_t count, int64_t M,
                                       uint16_t* const* dxs, float* const* dws,
                                       void* workspace, size_t workspace_bytes, void* stream);

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
