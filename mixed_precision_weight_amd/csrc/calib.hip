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
// Both sums are column reductions of an fp16 [R][K] matrix streamed from HBM.
// Kernel shape (HBM-bound): a 256-thread block owns a 64-column tile of one row
// slice. Lane (wave w, lane l) reads 8 columns (16 B) at column 8*(l%8) of rows
// w*8 + l/8 + 32 t, so each wave instruction reads 8 full 128-byte lines. Squares
// of fp16 values and of the (exact) fp32 RTN errors are accumulated in fp64; the
// 32 row phases are combined by a fixed butterfly and a fixed-order LDS sum,
// and row slices by a fixed-order final pass: results are bitwise deterministic.
//
// Built with -ffp-contract=off: the quantiser steps are single IEEE operations.
#include <mutex>

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

constexpr int kTileCols = 64;   // columns per block tile
constexpr int kPhases = 32;     // row phases per block (4 waves x 8)
constexpr int kUnroll = 4;      // rows in flight per lane

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

struct ErrElem {  // dW = w - s (q - z), exact in fp32; squared in fp64 by the caller
    const uint16_t* s16;
    const uint8_t* z;
    typedef RtnRow Row;
    __device__ __forceinline__ Row load_row(int64_t r) const { return make_rtn_row(h2f(s16[r]), z[r]); }
    __device__ __forceinline__ float val(const Row& rw, uint16_t h) const
    {
        // The residual against the (possibly clamped) grid point, exact: every
        // weight lies inside the row's full-row fit range, so |w / s| <= 8 and the
        // product of the offset and the 11-bit step has at most 14 bits. The
        // rounded quotient t = rint(w rs) is rint(w / s) except possibly at an
        // exact half-integer (see rint_quotient), where both neighbours leave
        // |residual| = s / 2, and the clamp to the code range maps an
        // out-of-range neighbour onto the in-range one; the squared residual is
        // therefore the same as with the tie rounded to even.
        const float w = h2f(h);
        const float q = __builtin_amdgcn_fmed3f(rintf(w * rw.rs), rw.lo, rw.hi);
        return __builtin_fmaf(-q, rw.s, w);
    }
    static constexpr bool kSquared = false;
};

// Column sums of one 64-column tile over one row slice, into partial[slice][.]
template <class Elem>
__device__ __forceinline__ void colsum_tile(const uint16_t* __restrict__ A, int64_t R, int64_t K,
                                            int64_t rows_per_slice, double* __restrict__ partial, Elem elem,
                                            int64_t tile, int64_t slice, double (&red)[4][kTileCols])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
    for (int64_t rb = r0 + phase; rb < r1; rb += (int64_t)kPhases * kUnroll) {
        uint4 v[kUnroll];
        typename Elem::Row rw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t r = min(rb + (int64_t)u * kPhases, r1 - 1);
            v[u] = *reinterpret_cast<const uint4*>(A + r * K + colc);
            rw[u] = elem.load_row(r);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            if (!(active && rb + (int64_t)u * kPhases < r1))
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
            t += red[1][threadIdx.x];
            t += red[2][threadIdx.x];
            t += red[3][threadIdx.x];
            partial[slice * K + j] = t;
        }
    }
}

// One wave per row: min/max over all K columns -> (fp16 step, zero point).
__device__ __forceinline__ void rowfit_rows(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                            uint16_t* __restrict__ s16, uint8_t* __restrict__ z, int64_t blk)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = blk * 4 + (threadIdx.x >> 6);
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

// First launch: the X column sums (lambda partials) and the W row fits run as
// one grid, tile-major X blocks first.
__global__ __launch_bounds__(256) void k_calib_first(const uint16_t* __restrict__ X, int64_t T, int64_t K,
                                                     int64_t rows_x, double* __restrict__ px, int64_t tiles,
                                                     int64_t nx, const uint16_t* __restrict__ W, int64_t N,
                                                     uint16_t* __restrict__ s16, uint8_t* __restrict__ z)
{
    __shared__ double red[4][kTileCols];
    const int64_t b = blockIdx.x;
    if (b < nx)
        colsum_tile(X, T, K, rows_x, px, SqElem{}, b % tiles, b / tiles, red);
    else
        rowfit_rows(W, N, K, s16, z, b - nx);
}

// Second launch: the RTN-error column sums over (tile, slice) blocks.
__global__ __launch_bounds__(256) void k_colsum_err(const uint16_t* __restrict__ W, int64_t N, int64_t K,
                                                    int64_t rows_w, double* __restrict__ pw, ErrElem elem)
{
    __shared__ double red[4][kTileCols];
    colsum_tile(W, N, K, rows_w, pw, elem, blockIdx.x, blockIdx.y, red);
}

// Third launch: lambda_j = 2 sum_s px[s][j], e_j = sum_s pw[s][j] (slices in
// order), score_j = lambda_j e_j. A separate launch: the slice partials come
// from blocks on all eight XCDs, whose L2 caches a device-wide fence would have
// to write back and invalidate.
__global__ __launch_bounds__(256) void k_finalize(const double* __restrict__ px, int64_t sx,
                                                  const double* __restrict__ pw, int64_t sw, int64_t K,
                                                  double* __restrict__ lambda, double* __restrict__ score)
{
    int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K)
        return;
    double l = 0.0;
#pragma unroll 8
    for (int64_t s = 0; s < sx; s++)
        l += px[s * K + j];
    l *= 2.0;
    double e = 0.0;
#pragma unroll 8
    for (int64_t s = 0; s < sw; s++)
        e += pw[s * K + j];
    lambda[j] = l;
    score[j] = l * e;
}

int64_t choose_slices(int64_t R, int64_t K)
{
    int64_t tiles = (K + kTileCols - 1) / kTileCols;
    int64_t s = (1024 + tiles - 1) / tiles;           // ~1024 blocks in flight
    int64_t cap = (R + 2 * kPhases - 1) / (2 * kPhases);  // >= 2 rows per phase
    if (s > cap)
        s = cap;
    if (s > 65535)
        s = 65535;
    return s < 1 ? 1 : s;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

CalibPlan calib_plan(int64_t N, int64_t K, int64_t T)
{
    CalibPlan p;
    p.sx = choose_slices(T, K);
    p.sw = choose_slices(N, K);
    p.rows_x = (T + p.sx - 1) / p.sx;
    p.rows_w = (N + p.sw - 1) / p.sw;
    size_t o = 0;
    p.off_px = o;
    o = align256(o + (size_t)p.sx * K * sizeof(double));
    p.off_pw = o;
    o = align256(o + (size_t)p.sw * K * sizeof(double));
    p.off_s16 = o;
    o = align256(o + (size_t)N * sizeof(uint16_t));
    p.off_z = o;
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

hipError_t launch_calibrate(const uint16_t* W, int64_t N, int64_t K, const uint16_t* X, int64_t T,
                            double* lambda, double* score, void* ws, const CalibPlan& p,
                            hipStream_t s)
{
    char* base = static_cast<char*>(ws);
    double* px = reinterpret_cast<double*>(base + p.off_px);
    double* pw = reinterpret_cast<double*>(base + p.off_pw);
    uint16_t* s16 = reinterpret_cast<uint16_t*>(base + p.off_s16);
    uint8_t* z = reinterpret_cast<uint8_t*>(base + p.off_z);
    const unsigned tiles = (unsigned)((K + kTileCols - 1) / kTileCols);

    const int64_t nx = (int64_t)tiles * p.sx;
    const int64_t nrow = (N + 3) / 4;
    hipLaunchKernelGGL(k_calib_first, dim3((unsigned)(nx + nrow)), dim3(256), 0, s, X, T, K, p.rows_x, px,
                       (int64_t)tiles, nx, W, N, s16, z);
    hipLaunchKernelGGL(k_colsum_err, dim3(tiles, (unsigned)p.sw), dim3(256), 0, s, W, N, K, p.rows_w, pw,
                       ErrElem{s16, z});
    hipLaunchKernelGGL(k_finalize, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s, px, p.sx, pw, p.sw, K,
                       lambda, score);
    return hipGetLastError();
}

}  // namespace owq
