// owq_launch.h -- host-side launchers of the gfx950 kernels (internal to libowq).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace owq {

// ---------------------------------------------------------------- calibrate --
struct CalibPlan {
    int64_t sx, sw;          // row slices of X and of W
    int64_t rows_x, rows_w;  // rows per slice
    size_t off_px, off_pw, off_s16, off_z, total;  // workspace byte offsets / size
};
CalibPlan calib_plan(int64_t N, int64_t K, int64_t T);
hipError_t launch_calibrate(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            double* lambda, double* score, void* ws, const CalibPlan& p,
                            hipStream_t s);

// ------------------------------------------------------------------- select --
hipError_t launch_select(const double* score, int64_t K, int32_t k, int32_t* idx, hipStream_t s);

// --------------------------------------------------------------------- pack --
hipError_t launch_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                       uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s);

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
// Matrix-core decode over `count` layers (count <= kGemvMaxLayers), 1 <= M <= kMfvMaxM.
constexpr int kMfvMaxM = 16;
hipError_t launch_mfv(const LinearDesc* d, int count, int M, hipStream_t s);
bool mfv_fits(int64_t M, int64_t K);
// Decode kernel choice for M tokens: true = matrix-core decode (launch_mfv), false =
// vector-ALU decode (launch_gemv). OWQ_DECODE=vector|matrix overrides (read per call).
bool decode_on_matrix_cores(int64_t M);
// Matrix-core GEMM for larger M.
hipError_t launch_gemm(const LinearDesc& d, int64_t M, hipStream_t s);

// read-only streaming reference (stream.hip): one word per 4608-byte wavefront
int64_t stream_read_sink_words(int64_t bytes);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
// Smallest M routed to the matrix-core kernel (read once from OWQ_GEMM_MIN_M).
int64_t gemm_min_m();

}  // namespace owq
