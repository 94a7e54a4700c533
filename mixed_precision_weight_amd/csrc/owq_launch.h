// owq_launch.h -- host-side launchers of the gfx950 kernels (internal to libowq).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace owq {

// ---------------------------------------------------------------- calibrate --
struct CalibPlan {
    int64_t sx, sw;          // row slices of X and of W (W: one per fused block)
    int64_t rows_x, rows_w;  // rows per slice
    int32_t wpl, nwaves;     // fused W form: 16-byte words per lane and waves per block; wpl 0: two-pass form
    size_t off_px, off_pw, off_s16, off_z, total;  // workspace byte offsets / size
};
CalibPlan calib_plan(int64_t N, int64_t K, int64_t T);
struct CalibItem {
    const uint16_t* W;
    int64_t N, K;
    const uint16_t* X;
    int64_t T;
    double* lambda;
    double* score;
};
// `count` calibrations in count + 2 launches (each linear's three passes
// staggered over three consecutive launches); ws[l]: item l's workspace of plan
// plans[l].
hipError_t launch_calibrate_batched(const CalibItem* items, int count, void* const* ws, const CalibPlan* plans,
                                   hipStream_t s);
hipError_t launch_calibrate(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            double* lambda, double* score, void* ws, const CalibPlan& p,
                            hipStream_t s);
// The library's own calibration workspace on the current device: a file-scope
// device array of kCalibScratchBytes (256-byte aligned), its address looked up
// once per device. Returns the HIP error of the lookup, if any.
constexpr size_t kCalibScratchBytes = (size_t)64 << 20;
hipError_t calib_scratch(void** ptr);

// ------------------------------------------------------------------- select --
hipError_t launch_select(const double* score, int64_t K, int32_t k, int32_t* idx, hipStream_t s);
// `count` selections (k[i] == 0 skipped): one block each, one launch per
// kSelectMaxBatch selections with the widest block shape among them (one
// launch per selection above K = 16384)
constexpr int kSelectMaxBatch = 64;
hipError_t launch_select_batched(const double* const* score, const int64_t* K, const int32_t* k,
                                 int32_t* const* idx, int count, hipStream_t s);

// --------------------------------------------------------------------- pack --
// one linear of a batched pack: owq_pack's arguments (idx, ww NULL when k == 0)
struct PackItem {
    const uint16_t* W;
    int64_t N, K;
    const int32_t* idx;
    int32_t k;
    uint32_t* q;
    uint16_t* scales;
    uint8_t* zeros;
    uint16_t* ww;
};
// linears per launch: those of one kernel form share a launch
constexpr int kPackMaxLayers = 16;
hipError_t launch_pack_batched(const PackItem* items, int count, hipStream_t s);
hipError_t launch_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                       uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s);
// The pack with each row's (step, zero point) read from scales / zeros.
hipError_t launch_pack_given(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                             uint32_t* q, const uint16_t* scales, const uint8_t* zeros, uint16_t* ww,
                             hipStream_t s);
// Truncation-aware (step, zero point) per row over its dense columns, written to
// scales / zeros (search.hip). lambda: fp64 [K] column weights, or NULL.
hipError_t launch_search(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                         const double* lambda, uint16_t* scales, uint8_t* zeros, hipStream_t s);

// ------------------------------------------------------------------- linear --
struct LinearDesc {
    const uint32_t* q;
    const uint16_t* s;
    const uint8_t* z;
    const int32_t* idx;
    const uint16_t* ww;
    const uint16_t* x;
    uint16_t* y;
    int64_t N, K;
    int32_t k;
    // x the weak columns are gathered from, with rows of kw columns (NULL: x and
    // K); the storage-favoured form gathers them from the full x while the dense
    // codes run against x at the dense columns (decode kernel on the vector ALUs only)
    const uint16_t* xw = nullptr;
    int64_t kw = 0;
};

constexpr int kGemvMaxM = 4;        // tokens per GEMV launch
constexpr int kVectorDecodeMaxM = 2;  // above this the matrix-core decode is faster (measured)
constexpr int kGemvMaxLayers = 16;  // layers per batched GEMV launch

// Decode GEMV over `count` layers (count <= kGemvMaxLayers), 1 <= M <= kGemvMaxM,
// gemv_fits(M, K) for every layer.
hipError_t launch_gemv(const LinearDesc* d, int count, int M, hipStream_t s);
// Tokens per GEMV launch for a layer of K columns (x of all tokens is staged in LDS).
int gemv_max_tokens(int64_t K);
bool gemv_fits(int64_t M, int64_t K);
// Products of the vector-ALU decode for M tokens: true = one v_mfma_f32_16x16x32_f16
// per token and 8 columns (M <= 2), false = v_dot2 per column pair.
// OWQ_GEMV_PRODUCTS=dot2|mfma overrides (read per call).
bool gemv_products_on_matrix_cores(int64_t M);
// Matrix-core decode over `count` layers (count <= kGemvMaxLayers), 1 <= M <= kMfvMaxM.
constexpr int kMfvMaxM = 16;
hipError_t launch_mfv(const LinearDesc* d, int count, int M, hipStream_t s);
bool mfv_fits(int64_t M, int64_t K);
// Decode kernel choice for M tokens: true = matrix-core decode (launch_mfv), false =
// vector-ALU decode (launch_gemv). OWQ_DECODE=vector|matrix overrides (read per call).
bool decode_on_matrix_cores(int64_t M);
// Group-wise form: a step and zero point per (row, group of G columns), G in
// {32, 64, ..., 2048} dividing K; scales / zeros [N][K/G].
bool grouped_size_supported(int64_t G, int64_t K);
hipError_t launch_pack_grouped(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k, int64_t G,
                               uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s);
// Group-wise decode of `count` layers (count <= kGemvMaxLayers) in one launch,
// 1 <= M <= kGemvMaxM tokens; groups[l]: columns per scale group of layer l.
hipError_t launch_gemv_grouped(const LinearDesc* d, const int64_t* groups, int count, int M, hipStream_t s);
// Matrix-core GEMM for larger M.
hipError_t launch_gemm(const LinearDesc& d, int64_t M, hipStream_t s);

// The linear on the latency-favoured form for any M: the GEMM from gemm_min_m()
// tokens, else the decode kernels in token slices (api.cpp).
hipError_t launch_linear_any(const LinearDesc& d, int64_t M, hipStream_t s);

// ------------------------------------------------------ storage-favoured form --
// Dense columns rounded up to whole groups; workspace bytes of the product.
int64_t storage_dense_cols32(int64_t K, int32_t k);
size_t storage_workspace_bytes(int64_t K, int32_t k, int64_t M);
hipError_t launch_pack_storage(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                               uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s);
// d: the layer with K its full column count and q its storage-form codes.
hipError_t launch_linear_storage(const LinearDesc& d, int64_t M, void* ws, hipStream_t s);
// `count` layers: three launches per kGemvMaxLayers layers (gathers, dense
// products, weak columns); ws[l]: layer l's workspace
hipError_t launch_linear_storage_batched(const LinearDesc* d, int count, int64_t M, void* const* ws, hipStream_t s);

// ------------------------------------------ backward (weak-column tuning) --
struct BwdPlan {
    int64_t slices, rows_per_slice;  // row slices of the transposed product (vector form, M <= 4)
    size_t off_p;                    // its partial sums
    // the matrix-core form (M > 4, 16 tokens per pass): row slices, partial
    // sums of the dense part and of the weak columns, the fp32 column sums
    int64_t m_slices, m_rows;
    size_t m_off_p, m_off_pw, m_off_f;
    size_t total;                    // workspace bytes (both forms share it)
};
BwdPlan bwd_plan(int64_t N, int64_t K, int32_t k);
// dx = dy W (fp16 [M][K], may be NULL) and dw_weak = dy^T x[:, idx] (fp32 [N][k],
// may be NULL); d.x is the layer input (read for dw), d.y unused.
hipError_t launch_linear_backward(const LinearDesc& d, const uint16_t* dy, int64_t M, uint16_t* dx, float* dw,
                                  void* ws, const BwdPlan& p, hipStream_t s);
// The same for `count` <= kBwdMaxLayers layers in one part launch and one
// finalize launch per 4-token chunk; dx[l] / dw[l] may be NULL, ws[l] is layer l's
// workspace (plan p[l]) when dx[l] is wanted.
constexpr int kBwdMaxLayers = 16;
hipError_t launch_linear_backward_batched(const LinearDesc* d, const uint16_t* const* dy, int count, int64_t M,
                                          uint16_t* const* dx, float* const* dw, void* const* ws,
                                          const BwdPlan* p, hipStream_t s);

// ------------------------------------------ OPTQ with the weak columns last --
struct OptqPlan {
    size_t off_perm, off_invr, off_h, off_mi, off_wc, off_err, off_qc, total;
};
OptqPlan optq_plan(int64_t N, int64_t K, int32_t k);
hipError_t launch_pack_optq(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            const int32_t* idx, int32_t k, uint32_t* q, uint16_t* scales, uint8_t* zeros,
                            uint16_t* ww, void* ws, const OptqPlan& p, hipStream_t s);

// read-only streaming reference (stream.hip): one word per 4608-byte wavefront
int64_t stream_read_sink_words(int64_t bytes);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
// Smallest M routed to the matrix-core kernel (read once from OWQ_GEMM_MIN_M).
int64_t gemm_min_m();

}  // namespace owq
