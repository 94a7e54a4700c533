// topk.hip -- weak-column selection: the k largest column scores (gfx950).
//
// The top-k columns by sensitivity become the weak columns kept in fp16 ([PL]
// "Weak-column selection", paper p.4; [PL] = paperlayer.ai page "OWQ:
// Outlier-Aware Weight Quantization for Efficient Fine-Tuning and Inference of
// Large Language Models"). Ties are broken by the lower column index and the
// result is written in ascending column order.
//
// One workgroup (latency-bound). For K <= 16384 the keys stay in registers
// (k_topk_reg, 512 or 1024 threads: early-exit radix select over the range the
// keys still in play span, one ordered prefix sum);
// larger K reads the scores from L2 on every pass (k_topk, below):
//  1. radix select of the k-th largest 64-bit order key, 8 bits per pass from the
//     most significant digit: an LDS histogram of the digit among keys that match
//     the digits fixed so far, then one wavefront scans the 256 bins;
//  2. one ordered compaction pass: column j is taken if its key is above the
//     threshold, or equal to it and among the first (k - #above) equal keys in
//     index order. Ballot/popcount scans keep index order, so the output is
//     ascending without a sort.
#include <algorithm>

#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

// Order-preserving map of a double to an unsigned key (+0 and -0 compare equal).
__device__ __forceinline__ uint64_t score_key(double v)
{
    if (v == 0.0)
        v = 0.0;
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t ballot)
{
    const int lane = threadIdx.x & 63;
    uint64_t m = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    return (uint32_t)__popcll(ballot & m);
}

// Exclusive block-wide prefix count of `flag` in thread order; also returns the total.
__device__ __forceinline__ uint32_t block_excl_count(bool flag, uint32_t* wave_tot, uint32_t& total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t b = __ballot(flag);
    if (lane == 0)
        wave_tot[wave] = (uint32_t)__popcll(b);
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < 16; w++) {
        uint32_t t = wave_tot[w];
        before += w < wave ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + lanes_below(b);
}

__global__ __launch_bounds__(1024) void k_topk(const double* __restrict__ score, int64_t K, int32_t k,
                                               int32_t* __restrict__ out)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wave_tot[16];
    __shared__ unsigned long long sh_prefix;
    __shared__ int sh_kk;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    uint64_t prefix = 0, mask = 0;
    int kk = k;  // how many still to take among keys matching `prefix` on `mask`
    for (int shift = 56; shift >= 0; shift -= 8) {
        if (tid < 256)
            hist[tid] = 0;
        __syncthreads();
        for (int64_t j = tid; j < K; j += 1024) {
            uint64_t key = score_key(score[j]);
            if ((key & mask) == prefix)
                atomicAdd(&hist[(key >> shift) & 255], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane l covers digits 255-4l .. 252-4l, i.e. descending order
            uint32_t c[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                c[i] = hist[255 - 4 * lane - i];
            uint32_t tot = c[0] + c[1] + c[2] + c[3];
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                uint32_t t = __shfl_up(incl, o, 64);
                if (lane >= o)
                    incl += t;
            }
            uint32_t excl = incl - tot;
            if (excl < (uint32_t)kk && incl >= (uint32_t)kk) {
                uint32_t run = excl;
                int d = 0;
                uint32_t above = 0;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (run + c[i] >= (uint32_t)kk) {
                        d = 255 - 4 * lane - i;
                        above = run;
                        break;
                    }
                    run += c[i];
                }
                sh_prefix = prefix | ((uint64_t)d << shift);
                sh_kk = kk - (int)above;
            }
        }
        __syncthreads();
        prefix = sh_prefix;
        kk = sh_kk;
        mask |= 0xffull << shift;
    }

    // ordered compaction: > threshold, or == threshold within the first kk in index order
    uint32_t base = 0, eq_base = 0;
    for (int64_t j0 = 0; j0 < K; j0 += 1024) {
        int64_t j = j0 + tid;
        uint64_t key = j < K ? score_key(score[j]) : 0;
        bool gt = j < K && key > prefix;
        bool eq = j < K && key == prefix;
        uint32_t eq_total;
        uint32_t eq_rank = eq_base + block_excl_count(eq, wave_tot, eq_total);
        bool sel = gt || (eq && eq_rank < (uint32_t)kk);
        uint32_t sel_total;
        uint32_t pos = base + block_excl_count(sel, wave_tot, sel_total);
        if (sel && pos < (uint32_t)k)
            out[pos] = (int32_t)j;
        base += sel_total;
        eq_base += eq_total;
    }
}

// Block-wide exclusive prefix sum of one value per thread (thread order) over
// NW waves; also returns the total. Two barriers.
template <int NW>
__device__ __forceinline__ uint32_t block_excl_sum(uint32_t v, uint32_t* wave_tot, uint32_t& total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o, 64);
        if (lane >= o)
            incl += t;
    }
    if (lane == 63)
        wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
    for (int w = 0; w < NW; w++) {
        const uint32_t t = wave_tot[w];
        before += w < wave ? t : 0;
        tot += t;
    }
    __syncthreads();
    total = tot;
    return before + incl - v;
}

// K <= 64 NW C: thread t holds the keys of columns C t .. C t + C - 1 in registers,
// so index order is thread order, then register order. The radix select works
// on the range [lo, hi] of the keys still in play, starting with the block's
// smallest and largest key: each pass splits it into 256 buckets of width 2^s
// (the smallest s that makes the range fit), so the first bucket boundaries
// follow the keys' actual spread rather than the fixed top byte (which for
// scores of similar magnitude holds a few values, and makes the waves' atomic
// counts collide). It stops as soon as the bucket holding the k-th key is taken
// whole, or when the bucket width is one (its keys are then equal). The
// selection is every key above the final range plus the first kk in index
// order inside it; one ordered prefix sum places it.
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m)
{
    const uint32_t a = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
    const uint32_t b = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
    return ((uint64_t)b << 32) | a;
}

template <int C, int NW>
__device__ __forceinline__ void topk_reg(const double* __restrict__ score, int32_t K, int32_t k,
                                         int32_t* __restrict__ out)
{
    __shared__ uint32_t hist[256];
    __shared__ uint32_t whist[NW][256];  // one digit histogram per wave
    __shared__ uint32_t wave_tot[NW];
    __shared__ unsigned long long sh_lo[NW], sh_hi[NW];
    __shared__ int sh_kk, sh_done;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (k <= 0)  // nothing to select (the host does not launch for k == 0)
        return;

    uint64_t key[C];
    uint64_t lo = ~0ull, hi = 0;
#pragma unroll
    for (int c = 0; c < C; c++) {
        const int j = C * tid + c;  // columns past K get key 0, below every finite score
        const double v = score[min(j, K - 1)];
        key[c] = j < K ? score_key(v) : 0ull;
        lo = j < K ? min(lo, key[c]) : lo;
        hi = j < K ? max(hi, key[c]) : hi;
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, shfl_xor_u64(lo, o));
        hi = max(hi, shfl_xor_u64(hi, o));
    }
    if (lane == 0) {
        sh_lo[wave] = lo;
        sh_hi[wave] = hi;
    }
    __syncthreads();
    lo = sh_lo[0];
    hi = sh_hi[0];
    for (int w = 1; w < NW; w++) {
        lo = min(lo, (uint64_t)sh_lo[w]);
        hi = max(hi, (uint64_t)sh_hi[w]);
    }
    __syncthreads();  // sh_lo / sh_hi are rewritten below

    int kk = k;  // how many still to take among the keys in [lo, hi]
    // each pass leaves a range at least 2^8 times narrower, so nine passes reach
    // width one; the bound only guarantees the loop ends
    for (int pass = 0; pass < 10; pass++) {
        const uint64_t span = hi - lo;
        const int s = span == 0 ? 0 : max(56 - (int)__clzll(span), 0);  // (span >> s) < 256
        // each wave counts its keys' buckets into its own LDS histogram (atomics
        // that hit one bin serialise within the wave only), then the 16 are summed
#pragma unroll
        for (int i = 0; i < 4; i++)
            whist[wave][lane + 64 * i] = 0;
#pragma unroll
        for (int c = 0; c < C; c++) {
            const uint64_t d = key[c] - lo;  // wraps above span for keys below lo
            if (d <= span)
                atomicAdd(&whist[wave][(uint32_t)(d >> s)], 1u);
        }
        __syncthreads();
        for (int b = tid; b < 256; b += 64 * NW) {
            uint32_t t = 0;
#pragma unroll
            for (int w = 0; w < NW; w++)
                t += whist[w][b];
            hist[b] = t;
        }
        __syncthreads();
        if (wave == 0) {
            // lane l covers buckets 255-4l .. 252-4l, i.e. descending order
            uint32_t c4[4];
#pragma unroll
            for (int i = 0; i < 4; i++)
                c4[i] = hist[255 - 4 * lane - i];
            const uint32_t tot = c4[0] + c4[1] + c4[2] + c4[3];
            uint32_t incl = tot;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t t = __shfl_up(incl, o, 64);
                if (lane >= o)
                    incl += t;
            }
            const uint32_t excl = incl - tot;
            if (excl < (uint32_t)kk && incl >= (uint32_t)kk) {
                uint32_t run = excl;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (run + c4[i] >= (uint32_t)kk) {
                        const uint64_t b0 = lo + ((uint64_t)(255 - 4 * lane - i) << s);
                        const uint64_t w = (1ull << s) - 1;
                        sh_lo[0] = b0;
                        sh_hi[0] = hi - b0 < w ? hi : b0 + w;
                        sh_kk = kk - (int)run;
                        // the whole bucket is taken, or its keys are all equal
                        sh_done = run + c4[i] == (uint32_t)kk || s == 0;
                        break;
                    }
                    run += c4[i];
                }
            }
        }
        __syncthreads();
        lo = sh_lo[0];
        hi = sh_hi[0];
        kk = sh_kk;
        const bool done = sh_done;
        __syncthreads();  // every thread has read the shared state before the next pass writes it
        if (done)
            break;
    }

    // ordered selection: above the final range, or inside it and among the first
    // kk such keys in index order
    const uint64_t span = hi - lo;
    uint32_t n_eq = 0;
#pragma unroll
    for (int c = 0; c < C; c++)
        n_eq += key[c] - lo <= span;
    uint32_t eq_total;
    uint32_t eq_rank = block_excl_sum<NW>(n_eq, wave_tot, eq_total);
    bool sel[C];
    uint32_t n_sel = 0;
#pragma unroll
    for (int c = 0; c < C; c++) {
        const bool eq = key[c] - lo <= span;
        sel[c] = key[c] > hi || (eq && eq_rank < (uint32_t)kk);
        eq_rank += eq;
        n_sel += sel[c];
    }
    uint32_t sel_total;
    uint32_t pos = block_excl_sum<NW>(n_sel, wave_tot, sel_total);
#pragma unroll
    for (int c = 0; c < C; c++)
        if (sel[c]) {
            if (pos < (uint32_t)k)
                out[pos] = C * tid + c;
            pos++;
        }
}

template <int C, int NW>
__global__ __launch_bounds__(64 * NW) void k_topk_reg(const double* __restrict__ score, int32_t K, int32_t k,
                                                      int32_t* __restrict__ out)
{
    topk_reg<C, NW>(score, K, k, out);
}

// several selections of one block shape, a block each
struct SelBatch {
    const double* score[kSelectMaxBatch];
    int32_t* out[kSelectMaxBatch];
    int32_t K[kSelectMaxBatch], k[kSelectMaxBatch];
    int32_t count;
};

template <int C, int NW>
__global__ __launch_bounds__(64 * NW) void k_topk_reg_batched(const SelBatch b)
{
    const int i = blockIdx.x;
    topk_reg<C, NW>(b.score[i], b.K[i], b.k[i], b.out[i]);
}

// the block shape for K <= 16384: 0 = 8 x 8 waves, 1 = 11 x 16, 2 = 16 x 16, 3 = k_topk
int shape_of(int64_t K) { return K <= 8 * 512 ? 0 : K <= 11 * 1024 ? 1 : K <= 16 * 1024 ? 2 : 3; }

}  // namespace

hipError_t launch_select_batched(const double* const* score, const int64_t* K, const int32_t* k,
                                 int32_t* const* idx, int count, hipStream_t s)
{
    auto flush = [&](int shape, SelBatch& b) {
        if (b.count == 0)
            return;
        if (shape == 0)
            hipLaunchKernelGGL((k_topk_reg_batched<8, 8>), dim3(b.count), dim3(512), 0, s, b);
        else if (shape == 1)
            hipLaunchKernelGGL((k_topk_reg_batched<11, 16>), dim3(b.count), dim3(1024), 0, s, b);
        else
            hipLaunchKernelGGL((k_topk_reg_batched<16, 16>), dim3(b.count), dim3(1024), 0, s, b);
        b.count = 0;
    };
    for (int i = 0; i < count; i++)  // large K: one launch each
        if (k[i] > 0 && shape_of(K[i]) == 3)
            hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), 0, s, score[i], K[i], k[i], idx[i]);
    // the register-path selections run side by side in one launch, with the
    // widest block shape any of them needs: the launch then takes about as long
    // as its slowest selection, where one launch per shape would add them up
    // (the selected set is unique, so the shape does not change a result)
    int shape = -1;
    for (int i = 0; i < count; i++)
        if (k[i] > 0 && shape_of(K[i]) < 3)
            shape = std::max(shape, shape_of(K[i]));
    SelBatch b{};
    for (int i = 0; i < count; i++) {
        if (k[i] == 0 || shape_of(K[i]) == 3)
            continue;
        b.score[b.count] = score[i];
        b.out[b.count] = idx[i];
        b.K[b.count] = (int32_t)K[i];
        b.k[b.count] = k[i];
        if (++b.count == kSelectMaxBatch)
            flush(shape, b);
    }
    flush(shape, b);
    return hipGetLastError();
}

hipError_t launch_select(const double* score, int64_t K, int32_t k, int32_t* idx, hipStream_t s)
{
    // block shapes measured on lognormal scores (one launch, HIP events): at
    // K = 4096 8 keys x 8 waves took 8.2 us against 10.4 / 9.7 / 12.1 us for
    // 4 x 16, 16 x 4 and 32 x 2; at K = 11008 11 x 16 took 14.9 us against
    // 17.2 / 15.2 / 18.6 us for 16 x 16, 22 x 8 and 43 x 4
    if (K <= 8 * 512)
        hipLaunchKernelGGL((k_topk_reg<8, 8>), dim3(1), dim3(512), 0, s, score, (int32_t)K, k, idx);
    else if (K <= 11 * 1024)
        hipLaunchKernelGGL((k_topk_reg<11, 16>), dim3(1), dim3(1024), 0, s, score, (int32_t)K, k, idx);
    else if (K <= 16 * 1024)
        hipLaunchKernelGGL((k_topk_reg<16, 16>), dim3(1), dim3(1024), 0, s, score, (int32_t)K, k, idx);
    else
        hipLaunchKernelGGL(k_topk, dim3(1), dim3(1024), 0, s, score, K, k, idx);
    return hipGetLastError();
}

}  // namespace owq
