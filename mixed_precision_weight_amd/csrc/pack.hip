// pack.hip -- latency-favoured OWQ storage of one layer (gfx950).
//
// The complete 3-bit matrix keeps zero-filled weak columns, and the weak
// columns are stored separately in fp16 ([PL] "Storage Methods", paper appendix
// section 2 pp.10-11). Weak columns are excluded from quantisation ([PL]
// "Weak-column selection", paper p.4), so each row is fitted on its dense
// columns; for an asymmetric grid, "zero-filled" is the zero-point code.
// [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models".
//
// Because the fitted range always contains 0, replacing the weak entries of a
// row by +0 leaves (lo, hi) of the dense columns unchanged and gives them the
// code clamp(rint(0/s) + z) = z. The kernel therefore zeroes the weak entries
// (a per-group 32-bit weak mask built once per block in LDS) and runs the plain
// full-row quantiser: one 256-thread block per row (grid-stride), each thread
// holding GPT 32-column groups in registers, a block min/max, then 32 codes per
// group packed into three words, the code of column c in slot kSlot[c] (bits
// [3 kSlot[c], 3 kSlot[c] + 3) of w0|w1<<32|w2<<64): columns 2p and 2p+1 take the
// p-th slot pair, (j, j+5) for j = 1..5, 11..15, 21..25, then (0, 31), so the
// decoders get both codes of a column pair from one 32-bit window.
//
// Built with -ffp-contract=off: the quantiser steps are single IEEE operations
// (the code itself comes from rint_quotient, which reproduces rint(w / s)
// exactly).
#include <algorithm>
#include <vector>

#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

// slot of column c within its 32-column group
constexpr int kSlot[32] = {1,  6,  2,  7,  3,  8,  4,  9,  5,  10, 11, 16, 12, 17, 13, 18,
                           14, 19, 15, 20, 21, 26, 22, 27, 23, 28, 24, 29, 25, 30, 0,  31};

// One launch packs up to kPackMaxLayers linears of one kernel form: blocks
// [b0[l], b0[l+1]) walk linear l's rows (grid-stride over that range).
struct PackLayer {
    const uint16_t* W;
    const int32_t* idx;
    uint32_t* q;
    uint16_t* scales;
    uint8_t* zeros;
    uint16_t* ww;
    int64_t N, K;
    int32_t k, pad;
};

struct PackBatch {
    PackLayer L[kPackMaxLayers];
    int32_t b0[kPackMaxLayers + 1];
    int32_t count;
};

__device__ __forceinline__ int pack_layer_of(const PackBatch& b)
{
    int l = 0;
    while (l + 1 < b.count && (int)blockIdx.x >= b.b0[l + 1])
        l++;
    return l;
}

// kGiven: each row's (step, zero point) is read from scales / zeros (written
// there before, e.g. by the truncation-aware search) instead of fitted.
template <int GPT, bool kGiven>
__global__ __launch_bounds__(256) void k_pack(const PackBatch b)
{
    const int li = pack_layer_of(b);
    const PackLayer& PL = b.L[li];
    const uint16_t* __restrict__ W = PL.W;
    const int64_t N = PL.N, K = PL.K;
    const int32_t* __restrict__ idx = PL.idx;
    const int32_t k = PL.k;
    uint32_t* __restrict__ q = PL.q;
    uint16_t* __restrict__ scales = PL.scales;
    uint8_t* __restrict__ zeros = PL.zeros;
    uint16_t* __restrict__ ww = PL.ww;
    const int64_t blk = (int64_t)blockIdx.x - b.b0[li], nblk = b.b0[li + 1] - b.b0[li];
    extern __shared__ uint32_t wmask[];  // [G] weak-column bit mask per 32-column group
    __shared__ float red[2][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t G = K / 32;

    for (int64_t g = tid; g < G; g += 256)
        wmask[g] = 0;
    __syncthreads();
    for (int64_t c = tid; c < k; c += 256) {
        const int32_t j = idx[c];
        if (j >= 0 && j < K)  // indices outside [0, K) break the caller contract; never touch memory with them
            atomicOr(&wmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();

    for (int64_t row = blk; row < N; row += nblk) {
        const uint16_t* wr = W + row * K;
        uint32_t v[GPT][16];
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int u = 0; u < GPT; u++) {
            int64_t g = tid + 256 * u;
            if (g < G) {
                const uint4* p = reinterpret_cast<const uint4*>(wr + g * 32);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    uint4 t = p[i];
                    v[u][4 * i + 0] = t.x;
                    v[u][4 * i + 1] = t.y;
                    v[u][4 * i + 2] = t.z;
                    v[u][4 * i + 3] = t.w;
                }
                uint32_t m = wmask[g];
#pragma unroll
                for (int c = 0; c < 32; c++) {
                    if ((m >> c) & 1u)
                        v[u][c >> 1] &= (c & 1) ? 0x0000ffffu : 0xffff0000u;
                    float f = h2f((uint16_t)(v[u][c >> 1] >> (16 * (c & 1))));
                    lo = fminf(lo, f);
                    hi = fmaxf(hi, f);
                }
            }
        }
        uint16_t s16;
        int z;
        if (kGiven) {
            s16 = scales[row];
            z = zeros[row];
        } else {
            lo = wave_min(lo);
            hi = wave_max(hi);
            if (lane == 0) {
                red[0][wave] = lo;
                red[1][wave] = hi;
            }
            __syncthreads();
            lo = fminf(fminf(red[0][0], red[0][1]), fminf(red[0][2], red[0][3]));
            hi = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
            qparams_from_range(lo, hi, s16, z);
        }
        const RtnRow rr = make_rtn_row(h2f(s16), z);
#pragma unroll
        for (int u = 0; u < GPT; u++) {
            int64_t g = tid + 256 * u;
            if (g < G) {
                uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
                for (int c = 0; c < 32; c++) {
                    uint32_t cd = (uint32_t)rtn_code(h2f((uint16_t)(v[u][c >> 1] >> (16 * (c & 1)))), rr);
                    const int pos = 3 * kSlot[c], wd = pos >> 5, off = pos & 31;
                    o[wd] |= cd << off;
                    if (off > 29)
                        o[wd + 1] |= cd >> (32 - off);
                }
                uint32_t* dst = q + (row * G + g) * 3;
                dst[0] = o[0];
                dst[1] = o[1];
                dst[2] = o[2];
            }
        }
        if (!kGiven && tid == 0) {
            scales[row] = s16;
            zeros[row] = (uint8_t)z;
        }
        for (int64_t c = tid; c < k; c += 256) {
            const int32_t j = idx[c];
            ww[row * k + c] = (j >= 0 && j < K) ? wr[j] : (uint16_t)0;
        }
        __syncthreads();  // red[] is reused by the next row
    }
}

// Wave-per-row form for K <= 64 GPW 32 (used up to 6144 columns): a wave holds its row's
// groups g = lane + 64 u in registers, so the row's min/max is a wave reduction
// and no block barrier separates the load from the codes; a block of 4 waves
// walks 4 rows at a time (grid-stride). Lanes write their groups' 12 bytes next
// to each other, 768 contiguous bytes per store instruction.
template <int GPW, bool kGiven>
__global__ __launch_bounds__(256) void k_pack_w(const PackBatch b)
{
    const int li = pack_layer_of(b);
    const PackLayer& PL = b.L[li];
    const uint16_t* __restrict__ W = PL.W;
    const int64_t N = PL.N, K = PL.K;
    const int32_t* __restrict__ idx = PL.idx;
    const int32_t k = PL.k;
    uint32_t* __restrict__ q = PL.q;
    uint16_t* __restrict__ scales = PL.scales;
    uint8_t* __restrict__ zeros = PL.zeros;
    uint16_t* __restrict__ ww = PL.ww;
    const int64_t blk = (int64_t)blockIdx.x - b.b0[li], nblk = b.b0[li + 1] - b.b0[li];
    extern __shared__ uint32_t wmask[];  // [G] weak-column bit mask per 32-column group
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (int)(K / 32);

    for (int g = tid; g < G; g += 256)
        wmask[g] = 0;
    __syncthreads();
    for (int c = tid; c < k; c += 256) {
        const int32_t j = idx[c];
        if (j >= 0 && j < K)  // indices outside [0, K) break the caller contract; never touch memory with them
            atomicOr(&wmask[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    uint32_t m[GPW];
#pragma unroll
    for (int u = 0; u < GPW; u++)
        m[u] = wmask[min(lane + 64 * u, G - 1)];

    for (int64_t row = blk * 4 + wave; row < N; row += nblk * 4) {
        const uint16_t* wr = W + row * K;
        uint32_t v[GPW][16];
        // every load first (clamped to the row), then the weak entries zeroed
#pragma unroll
        for (int u = 0; u < GPW; u++) {
            const uint4* p = reinterpret_cast<const uint4*>(wr + (int64_t)min(lane + 64 * u, G - 1) * 32);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint4 t = p[i];
                v[u][4 * i + 0] = t.x;
                v[u][4 * i + 1] = t.y;
                v[u][4 * i + 2] = t.z;
                v[u][4 * i + 3] = t.w;
            }
        }
        // zero the weak entries: the two mask bits of a dword become the halves
        // of an AND mask (bit 0 -> low half, bit 1 -> high half); groups past K
        // are zeroed whole. Then min/max over the fp16 pairs (exact).
        half2_t lo2 = {(_Float16)0.0f, (_Float16)0.0f}, hi2 = lo2;
#pragma unroll
        for (int u = 0; u < GPW; u++) {
            const uint32_t mk = lane + 64 * u < G ? m[u] : 0xffffffffu;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const uint32_t k0 = (uint32_t)((int32_t)(mk << (31 - 2 * i)) >> 31);  // bit 2i spread
                const uint32_t k1 = (uint32_t)((int32_t)(mk << (30 - 2 * i)) >> 31);  // bit 2i + 1 spread
                v[u][i] &= ~((k0 & 0x0000ffffu) | (k1 & 0xffff0000u));
                const half2_t h = __builtin_bit_cast(half2_t, v[u][i]);
                lo2 = __builtin_elementwise_min(lo2, h);
                hi2 = __builtin_elementwise_max(hi2, h);
            }
        }
        uint16_t s16;
        int z;
        if (kGiven) {
            s16 = scales[row];
            z = zeros[row];
        } else {
            const float lo = wave_min(fminf((float)lo2.x, (float)lo2.y));
            const float hi = wave_max(fmaxf((float)hi2.x, (float)hi2.y));
            qparams_from_range(lo, hi, s16, z);
        }
        const RtnRow rr = make_rtn_row(h2f(s16), z);
#pragma unroll
        for (int u = 0; u < GPW; u++) {
            const int g = lane + 64 * u;
            uint32_t o[3] = {0u, 0u, 0u};
#pragma unroll
            for (int c = 0; c < 32; c++) {
                const uint32_t cd = (uint32_t)rtn_code(h2f((uint16_t)(v[u][c >> 1] >> (16 * (c & 1)))), rr);
                const int pos = 3 * kSlot[c], wd = pos >> 5, off = pos & 31;
                o[wd] |= cd << off;
                if (off > 29)
                    o[wd + 1] |= cd >> (32 - off);
            }
            if (g < G) {
                uint32_t* dst = q + (row * G + g) * 3;
                dst[0] = o[0];
                dst[1] = o[1];
                dst[2] = o[2];
            }
        }
        if (!kGiven && lane == 0) {
            scales[row] = s16;
            zeros[row] = (uint8_t)z;
        }
        for (int c = lane; c < k; c += 64) {
            const int32_t j = idx[c];
            ww[row * k + c] = (j >= 0 && j < K) ? wr[j] : (uint16_t)0;
        }
    }
}

// The kernel form of a linear: 1, 2, 3 = a wave per row with that many groups
// per lane; 4 + t = a block per row with 1, 2, 4, 8 groups per thread (t = 0..3).
int pack_form(int64_t K)
{
    const int64_t G = K / 32;
    // a wave per row while a lane's groups fit in registers with room to spare
    // (measured: K = 4096 17.5 us vs 20 us a block per row; at K = 11008 the
    // block form is faster)
    const int64_t gpw = (G + 63) / 64;  // groups per lane with a wave per row
    if (gpw <= 3)
        return (int)gpw;
    const int64_t gpt = (G + 255) / 256;  // K <= 65536 -> gpt <= 8
    return gpt <= 1 ? 4 : gpt <= 2 ? 5 : gpt <= 4 ? 6 : 7;
}

template <bool kGiven>
void launch_pack_form(int form, const PackBatch& b, size_t lds, hipStream_t s)
{
    const dim3 grid((unsigned)b.b0[b.count]), block(256);
    switch (form) {
    case 1: hipLaunchKernelGGL((k_pack_w<1, kGiven>), grid, block, lds, s, b); break;
    case 2: hipLaunchKernelGGL((k_pack_w<2, kGiven>), grid, block, lds, s, b); break;
    case 3: hipLaunchKernelGGL((k_pack_w<3, kGiven>), grid, block, lds, s, b); break;
    case 4: hipLaunchKernelGGL((k_pack<1, kGiven>), grid, block, lds, s, b); break;
    case 5: hipLaunchKernelGGL((k_pack<2, kGiven>), grid, block, lds, s, b); break;
    case 6: hipLaunchKernelGGL((k_pack<4, kGiven>), grid, block, lds, s, b); break;
    default: hipLaunchKernelGGL((k_pack<8, kGiven>), grid, block, lds, s, b); break;
    }
}

// Linears of one kernel form share a launch, kPackMaxLayers at a time. Blocks
// per linear: a wave-per-row block takes 4 rows per step, at most 2048 blocks;
// a block-per-row block one row, at most 4096 blocks (grid-stride beyond).
template <bool kGiven>
hipError_t launch_pack_batched_any(const PackItem* items, int count, hipStream_t s)
{
    std::vector<char> done((size_t)count, 0);
    for (int l0 = 0; l0 < count; l0++) {
        if (done[l0])
            continue;
        const int form = pack_form(items[l0].K);
        PackBatch b{};
        size_t lds = 0;
        auto flush = [&]() {
            if (b.count > 0)
                launch_pack_form<kGiven>(form, b, lds, s);
            b.count = 0;
            lds = 0;
        };
        for (int l = l0; l < count; l++) {
            if (done[l] || pack_form(items[l].K) != form)
                continue;
            done[l] = 1;
            const PackItem& it = items[l];
            PackLayer& L = b.L[b.count];
            L = PackLayer{it.W, it.idx, it.q, it.scales, it.zeros, it.ww, it.N, it.K, it.k, 0};
            const int64_t nb = form <= 3 ? std::min<int64_t>((it.N + 3) / 4, 2048) : std::min<int64_t>(it.N, 4096);
            b.b0[0] = 0;
            b.b0[b.count + 1] = b.b0[b.count] + (int32_t)nb;
            lds = std::max(lds, (size_t)(it.K / 32) * sizeof(uint32_t));
            if (++b.count == kPackMaxLayers)
                flush();
        }
        flush();
    }
    return hipGetLastError();
}

template <bool kGiven>
hipError_t launch_pack_any(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                           uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s)
{
    const PackItem it{W, N, K, idx, k, q, scales, zeros, ww};
    return launch_pack_batched_any<kGiven>(&it, 1, s);
}

}  // namespace

hipError_t launch_pack_batched(const PackItem* items, int count, hipStream_t s)
{
    return launch_pack_batched_any<false>(items, count, s);
}

hipError_t launch_pack(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                       uint32_t* q, uint16_t* scales, uint8_t* zeros, uint16_t* ww, hipStream_t s)
{
    return launch_pack_any<false>(W, N, K, idx, k, q, scales, zeros, ww, s);
}

hipError_t launch_pack_given(const uint16_t* W, int64_t N, int64_t K, const int32_t* idx, int32_t k,
                             uint32_t* q, const uint16_t* scales, const uint8_t* zeros, uint16_t* ww,
                             hipStream_t s)
{
    // the kernels only read scales / zeros in this form
    return launch_pack_any<true>(W, N, K, idx, k, q, const_cast<uint16_t*>(scales), const_cast<uint8_t*>(zeros),
                                 ww, s);
}

}  // namespace owq
