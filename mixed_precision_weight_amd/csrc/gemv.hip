// gemv.hip -- decode-time OWQ linear, small batch M (gfx950, vector-ALU decode).
//
//   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
//
// The 3-bit dense matrix is streamed once from HBM; the weak fp16 block is a
// small contiguous [N][k] array and only x is gathered at the weak indices, on
// the fly ([PL] "Real-device acceleration", paper "Acceleration on Real Device"
// p.6; [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models").
//
// Work split: a block of 4 wavefronts owns 4 R consecutive rows of one layer
// (R rows per wavefront); the 64 lanes of a wave split a row's K/32 groups, lane
// l taking groups l, l + 64, ... (a "tile" is one 12-byte group per lane: 768
// contiguous bytes of one row). K is walked in chunks of two tiles (4096
// columns): for each chunk the block stages x in LDS in natural column order, every
// wave holds its R rows' code tiles in registers, and all global loads of the
// chunk are issued before the first wait (unconditionally, with clamped
// indices: a load under a divergent branch would make the compiler wait for it
// at the branch merge). The hardware overlaps the arithmetic of resident blocks
// with the loads of others. Layers of any K share the kernel, so the decode of a
// whole decoder layer (several linears) is one launch. Rows finish with a
// 64-lane reduction of up to four rows at once (lane-half swaps, then DPP).
//
// Each 12-byte group is decoded in registers (owq_decode.h) to sixteen exact
// (q_a - z, q_b - z) fp16 pairs of consecutive columns, and one v_dot2_f32_f16
// per pair multiplies it with the matching x dword, staged as stored. Every product is
// exact, so the fp32 sum's error is bounded relative to sum_j |(q_j - z) x_j|,
// for every row, including rows whose codes all equal the zero point. Per tile:
// 5 window ops, 17 and-or, 16 packed subtracts, 16 dot2 per token.
//
// With two tokens the dot2 work doubles, and the products move to the matrix
// cores instead: v_mfma_f32_16x16x32_f16 pairs the 8 A and the 8 B elements of
// each lane with the same 8 k indices, for A row and B column l % 16, so entry
// (i, i) of its 16 x 16 result is the sum, over lanes i, i + 16, i + 32 and
// i + 48, of each lane's own 8 decoded values times its own 8 x values. One MFMA
// per token and 8 columns (A = the lane's x quad, B = four decode pairs) keeps
// the lane layout, the loads and the staging of the vector form; the diagonal
// is read out at the end (15 of 16 results are discarded, the matrix cores have
// the throughput to spare) and the 64-lane reduction follows as before. The
// products stay exact and are summed in fp32. Lanes past a chunk's groups meet
// x staged as zeros.
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "owq_decode.h"
#include "owq_device.h"
#include "owq_launch.h"

namespace owq {

namespace {

struct GemvLayer {
    const uint32_t* q;
    const uint16_t* s;
    const uint8_t* z;
    const int32_t* idx;
    const uint16_t* ww;
    const uint16_t* x;
    uint16_t* y;
    int32_t N, K, k;
    int32_t block0;  // first block of this layer
    int32_t gsh;     // group-wise form: log2 of the 32-column code groups per scale group
    const uint16_t* xw;  // x of the weak columns (x itself, or the full x of the storage-favoured form)
    int32_t kw;          // its row length
};

struct GemvBatch {
    GemvLayer L[kGemvMaxLayers];
    int32_t count;
};

// Staged x layout (uint4 units): [m][tile u][quad qd][lane l] for group g = 64 u + l,
// so a lane's four quads of a tile are at immediate offsets and the lanes of a
// wave read consecutive 16-byte words. The quads are 68 slots apart: the
// staging writes, which take consecutive 16-byte pieces of x (group g / 4, quad
// g % 4 per lane), then spread over all 64 banks.
constexpr int kQuadStride = 68;
__device__ __forceinline__ int xs_slot(int m, int T, int g, int qd)
{
    return (m * T + (g >> 6)) * (4 * kQuadStride) + qd * kQuadStride + (g & 63);
}

// ------------------------------------------------------------------ kernel --
constexpr int kChunkTiles = 2;  // 64-group tiles per K chunk (4096 columns)
constexpr int kNonTemporal = 2;  // buffer-load cache-policy bits: nt
// Rows per wavefront: three (71 registers at M = 1, seven waves per SIMD) was
// faster than two, four (109 registers, four waves) and eight at M = 1 and 2.
constexpr int kRowsPerWave = 3;
// Below this many three-row blocks (one linear of a 7B layer: 342-918; the
// layer's 7 in one launch: 3,543) one token runs two rows per wave: measured
// 38.9-39.1 against 42.2-42.3 us for the 7 linears as 7 launches, and 21.1
// against 20.4-20.6 us for them in one launch
constexpr int kSmallLaunchBlocks = 1024;

__device__ __forceinline__ float f_of(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t u_of(float v) { return __builtin_bit_cast(uint32_t, v); }

// Sum over the 64 lanes of 4 per-lane values at once: a v_permlane32_swap and a
// v_permlane16_swap step each add two values while halving their lane span, then
// a DPP reduction inside 16-lane rows. On return a[0] holds, in lanes
// 16 q .. 16 q + 15, the total of input reduced_index(q).
__device__ __forceinline__ void reduce4(float (&a)[4])
{
    float b[2];
#pragma unroll
    for (int i = 0; i < 2; i++) {  // lanes 0-31 keep input i, lanes 32-63 input i + 2
        auto t = __builtin_amdgcn_permlane32_swap(u_of(a[i]), u_of(a[i + 2]), false, false);
        b[i] = f_of(t[0]) + f_of(t[1]);
    }
    auto t = __builtin_amdgcn_permlane16_swap(u_of(b[0]), u_of(b[1]), false, false);
    float v = f_of(t[0]) + f_of(t[1]);
    v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);  // row_ror:4
    v += dpp_f<0x128>(v);  // row_ror:8
    a[0] = v;
}
// quarter q of the lanes holds input (q & 1) + 2 (q >> 1)
__device__ __forceinline__ int reduced_index(int q) { return (q & 1) + ((q >> 1) << 1); }

// One wavefront computes R consecutive rows of one layer; a block is 4 waves
// (4 R rows) sharing x, staged in LDS in natural column order one K chunk
// (kChunkTiles tiles, 4096 columns) at a time. For each chunk every global load
// of the block (x of the chunk, the R rows' codes of the chunk, and with the
// first chunk the rows' scale, zero point, weak weights and the weak indices)
// is issued before the first wait, so a chunk costs one memory latency; the
// hardware overlaps the arithmetic of resident blocks with the loads of others.
// Layers of any K share this one kernel, so a batch is a single launch.
// GRP: the group-wise form (s and z are [N][K / G], one per row and G columns):
// each code group is decoded with its own zero point, its dot2 sum starts from 0
// and is scaled by its group's step into the row's accumulator.
template <int M, bool MMA, int R, bool GRP = false>
__device__ __forceinline__ void gemv_body(const GemvBatch& b)
{
    static_assert(!(GRP && MMA), "the group-wise form scales each lane's partial sum");
    constexpr int TT = kChunkTiles;
    constexpr int GC = 64 * TT;  // groups per chunk
    extern __shared__ uint4 smem[];
    int li = 0;
    for (int l = 1; l < b.count; l++)
        if ((int)blockIdx.x >= b.L[l].block0)
            li = l;
    const uint16_t* __restrict__ X = b.L[li].x;
    const int32_t* __restrict__ IDX = b.L[li].idx;
    const uint16_t* __restrict__ WW = b.L[li].ww;
    const uint16_t* __restrict__ XW = b.L[li].xw;
    const int N = b.L[li].N, K = b.L[li].K, k = b.L[li].k, KW = b.L[li].kw;
    const int G = K >> 5;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int brow = ((int)blockIdx.x - b.L[li].block0) * 4 * R;
    const int row0 = brow + wave * R;     // this wave's first row
    const int nb = min(N - brow, 4 * R);  // valid rows of the block

    // codes of the block's rows: raw buffer loads addressed by the per-lane offset
    // (which the range check covers), so bytes past the block's valid rows read 0
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(b.L[li].q) + (int64_t)brow * G * 3, (short)0, nb * G * 12, 0x00020000);
    int vrow[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        vrow[r] = (wave * R + r) * G * 12 + lane * 12;

    constexpr int PC = 4 * GC;        // 16-byte pieces of x per token and chunk
    constexpr int XP = M * PC / 256;  // staged pieces per thread
    uint4 xg[XP];
    u32x3 cw[R][TT];
    uint32_t zq[GRP ? R : 1][GRP ? TT : 1], sq[GRP ? R : 1][GRP ? TT : 1];  // group-wise zero points, steps
    const int gsh = b.L[li].gsh;
    const int NGS = G >> gsh;  // scale groups per row
    // Every load below is unconditional (indices clamped to valid data): a load
    // under a divergent branch makes the compiler wait for it before the branch
    // merges, which would serialise the x latency in front of the code loads.
    // Staging item i = m PC + p: token m, piece p of the chunk (consecutive
    // threads read consecutive 16 bytes of x).
    auto issue_chunk = [&](int g0, int gc) {
#pragma unroll
        for (int t = 0; t < XP; t++) {
            const int i = tid + 256 * t;
            const int m = i / PC, pc = min(i % PC, 4 * gc - 1);
            xg[t] = *reinterpret_cast<const uint4*>(X + m * K + g0 * 32 + pc * 8);
        }
        asm volatile("" ::: "memory");  // x ahead of the codes: its wait covers no code load
        // the codes are read once per launch: non-temporal loads (cache policy
        // "nt") keep them from displacing x and the row data in the caches
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int u = 0; u < TT; u++)
                cw[r][u] = __builtin_amdgcn_raw_buffer_load_b96(qr, vrow[r] + (g0 + 64 * u) * 12, 0, kNonTemporal);
        if constexpr (GRP) {
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int64_t base = (int64_t)min(row0 + r, N - 1) * NGS;
#pragma unroll
                for (int u = 0; u < TT; u++) {
                    const int gi = min(g0 + 64 * u + lane, G - 1) >> gsh;
                    zq[r][u] = b.L[li].z[base + gi];
                    sq[r][u] = b.L[li].s[base + gi];
                }
            }
        }
    };

    // row steps and zero points first: they move to scalar registers below, and
    // waiting for them then waits for nothing issued later
    uint32_t sv[R], zv[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = min(row0 + r, N - 1);
        sv[r] = GRP ? 0x3c00u : b.L[li].s[row];  // the group-wise form scales per group instead
        zv[r] = GRP ? 0u : b.L[li].z[row];
    }
    const int kc = k > 0 ? k : 1;  // with k == 0 the host passes valid dummy arrays
    int widx[2];  // weak indices: loaded early, so the gather's wait covers no code load
#pragma unroll
    for (int v = 0; v < 2; v++)
        widx[v] = IDX[min(lane + 64 * v, kc - 1)];
    asm volatile("" ::: "memory");  // keep them ahead of the chunk's loads
    issue_chunk(0, min(GC, G));
    // weak weights; x at the weak indices
    float wwv[R][2];
#pragma unroll
    for (int r = 0; r < R; r++) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int v = 0; v < 2; v++) {
            const int c = lane + 64 * v;
            const float w = h2f(WW[(int64_t)row * k + min(c, kc - 1)]);
            wwv[r][v] = c < k ? w : 0.0f;
        }
    }
    float xw[M][2];
#pragma unroll
    for (int v = 0; v < 2; v++) {
        const int c = lane + 64 * v;
        int j = widx[v];
        j = (j >= 0 && j < KW) ? j : 0;
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float xv = h2f(XW[(int64_t)m * KW + j]);
            xw[m][v] = c < k ? xv : 0.0f;
        }
    }

    float sc[R];
    uint32_t zr[R];
#pragma unroll
    for (int r = 0; r < R; r++) {
        sc[r] = h2f((uint16_t)__builtin_amdgcn_readfirstlane((int)sv[r]));
        zr[r] = (uint32_t)__builtin_amdgcn_readfirstlane((int)zv[r]);
    }

    const Magic mg = make_magic();
    float acc[R][M];
    float4_t macc[MMA ? R : 1][MMA ? M : 1];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            acc[r][m] = 0.0f;
            if (MMA)
                macc[r][m] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }

    for (int g0 = 0; g0 < G; g0 += GC) {
        const int gc = min(GC, G - g0);
        if (g0 > 0) {
            __syncthreads();  // every wave is done with the previous chunk's x
            issue_chunk(g0, gc);
        }
#pragma unroll
        for (int t = 0; t < XP; t++) {
            const int i = tid + 256 * t;
            const int pc = i % PC;
            if (MMA) {  // every slot is written: x, or zeros past the chunk's groups
                const bool on = pc < 4 * gc;
                smem[xs_slot(i / PC, TT, pc >> 2, pc & 3)] =
                    make_uint4(on ? xg[t].x : 0u, on ? xg[t].y : 0u, on ? xg[t].z : 0u, on ? xg[t].w : 0u);
            } else if (pc < 4 * gc) {
                smem[xs_slot(i / PC, TT, pc >> 2, pc & 3)] = make_uint4(xg[t].x, xg[t].y, xg[t].z, xg[t].w);
            }
        }
        __syncthreads();
        // x of a tile is read from LDS once (all four quads in flight together)
        // and shared by the R rows; lanes past the chunk's groups skip the rows
#pragma unroll
        for (int u = 0; u < TT; u++) {
            const int g = (u << 6) + lane;  // group within the chunk
            uint4 xq[M][4];
            if (!MMA) {
#pragma unroll
                for (int m = 0; m < M; m++)
#pragma unroll
                    for (int qd = 0; qd < 4; qd++)
                        xq[m][qd] = smem[xs_slot(m, TT, g, qd)];
            }
            if (MMA) {
                // lanes past the chunk's groups meet zeros in x: their products are 0.
                // Quad qd of x (columns 8 qd .. 8 qd + 7 of the lane's group) meets
                // decode pairs 4 qd .. 4 qd + 3 of each row.
                auto quad = [&](auto qdc) {
                    constexpr int qd = decltype(qdc)::value;
                    uint4 xv[M];
#pragma unroll
                    for (int m = 0; m < M; m++)
                        xv[m] = smem[xs_slot(m, TT, g, qd)];
#pragma unroll
                    for (int r = 0; r < R; r++) {
                        const ZeroSub nz = make_zero_sub(zr[r]);
                        uint32_t p[4];
                        decode_quad<qd>(cw[r][u].x, cw[r][u].y, cw[r][u].z, mg, nz, p);
                        const half8_t bq = __builtin_bit_cast(half8_t, make_uint4(p[0], p[1], p[2], p[3]));
#pragma unroll
                        for (int m = 0; m < M; m++)
                            macc[r][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                __builtin_bit_cast(half8_t, xv[m]), bq, macc[r][m], 0, 0, 0);
                    }
                };
                quad(std::integral_constant<int, 0>{});
                quad(std::integral_constant<int, 1>{});
                quad(std::integral_constant<int, 2>{});
                quad(std::integral_constant<int, 3>{});
            } else if (g < gc) {
#pragma unroll
                for (int r = 0; r < R; r++) {
                    const ZeroSub nz = make_zero_sub(GRP ? zq[r][u] : zr[r]);
                    uint32_t p[16];
                    decode_group(cw[r][u].x, cw[r][u].y, cw[r][u].z, mg, nz, p);
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        float a = GRP ? 0.0f : acc[r][m];
#pragma unroll
                        for (int qd = 0; qd < 4; qd++) {
                            a = dot2(p[4 * qd + 0], xq[m][qd].x, a);
                            a = dot2(p[4 * qd + 1], xq[m][qd].y, a);
                            a = dot2(p[4 * qd + 2], xq[m][qd].z, a);
                            a = dot2(p[4 * qd + 3], xq[m][qd].w, a);
                        }
                        acc[r][m] = GRP ? __builtin_fmaf(h2f((uint16_t)sq[r][u]), a, acc[r][m]) : a;
                    }
                }
            }
        }
    }

    if (MMA) {
        // The MFMA pairs lane l's A and B elements with the same k index, for A row
        // and B column l % 16: entry (i, i) of the 16 x 16 result sums the products
        // of lanes i, i + 16, i + 32 and i + 48 with their own x, i.e. of their own
        // groups. Entry (i, i) is element i % 4 of lane 16 (i / 4) + i; the other
        // entries pair one lane's codes with another lane's x and are dropped.
        const bool diag = (lane >> 4) == ((lane & 15) >> 2);
        const int e = lane & 3;
#pragma unroll
        for (int r = 0; r < R; r++)
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float4_t c = macc[r][m];
                const float v = e == 0 ? c[0] : e == 1 ? c[1] : e == 2 ? c[2] : c[3];
                acc[r][m] = diag ? v : 0.0f;
            }
    }

    // rows: scale, weak columns, 64-lane reduction of the rows together, fp16 store
    uint16_t* __restrict__ Y = b.L[li].y;
#pragma unroll
    for (int m = 0; m < M; m++) {
        constexpr int RQ = (R + 3) / 4;  // groups of four rows reduced together
        float part[RQ][4];
#pragma unroll
        for (int r = 0; r < 4 * RQ; r++) {
            part[r / 4][r % 4] = 0.0f;
            if (r < R) {
                float t = sc[r] * acc[r][m];
#pragma unroll
                for (int v = 0; v < 2; v++)
                    t += wwv[r][v] * xw[m][v];
                part[r / 4][r % 4] = t;
            }
        }
        if (k > 128) {  // remaining weak columns from global memory
#pragma unroll
            for (int r = 0; r < R; r++) {
                const int row = min(row0 + r, N - 1);
                for (int c = lane + 128; c < k; c += 64) {
                    int j = IDX[c];
                    j = (j >= 0 && j < KW) ? j : 0;
                    part[r / 4][r % 4] += h2f(WW[(int64_t)row * k + c]) * h2f(XW[(int64_t)m * KW + j]);
                }
            }
        }
#pragma unroll
        for (int qg = 0; qg < RQ; qg++) {
            reduce4(part[qg]);
            const int rr = 4 * qg + reduced_index(lane >> 4);
            if ((lane & 15) == 0 && rr < R && row0 + rr < N)
                Y[(int64_t)m * N + row0 + rr] = f2h(part[qg][0]);
        }
    }
}

template <int M>
__global__ __launch_bounds__(256) void k_gemv(GemvBatch b) { gemv_body<M, false, kRowsPerWave>(b); }
// one token, two rows per wave: for launches too small to fill the GPU with
// three-row waves (a single linear), half as many rows per block again
__global__ __launch_bounds__(256) void k_gemv_r2(GemvBatch b) { gemv_body<1, false, 2>(b); }
// the matrix-core products at five waves per SIMD (95 registers, no spills);
// without the occupancy bound the compiler takes 138 and runs three
template <int M>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_gemv_mfma(GemvBatch b)
{
    gemv_body<M, true, kRowsPerWave>(b);
}

// (97 registers at one token, four waves per SIMD: an occupancy bound of five
// or six spills)
template <int M>
__global__ __launch_bounds__(256) void k_gemv_grouped(GemvBatch b)
{
    gemv_body<M, false, kRowsPerWave, true>(b);
}

template <int M>
hipError_t launch_m(const GemvBatch& b, int nblocks, size_t lds, hipStream_t s)
{
    if constexpr (M <= 2) {
        if (gemv_products_on_matrix_cores(M)) {
            hipLaunchKernelGGL((k_gemv_mfma<M>), dim3(nblocks), dim3(256), lds, s, b);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((k_gemv<M>), dim3(nblocks), dim3(256), lds, s, b);
    return hipGetLastError();
}

}  // namespace

bool gemv_products_on_matrix_cores(int64_t M)
{
    const char* e = std::getenv("OWQ_GEMV_PRODUCTS");
    if (e && std::strcmp(e, "dot2") == 0)
        return false;
    if (e && std::strcmp(e, "mfma") == 0)
        return M <= 2;
    return M == 2;
}

int gemv_max_tokens(int64_t K)
{
    (void)K;
    return kGemvMaxM;
}

bool gemv_fits(int64_t M, int64_t K)
{
    (void)K;
    return M >= 1 && M <= kGemvMaxM;
}

namespace {

// The launch arguments of a batch (layers with the longest rows first: their
// blocks run longest); groups: the group-wise form's columns per scale group,
// per layer, or NULL for the per-row form. Returns the block count.
int build_batch(const LinearDesc* d, int count, const int64_t* groups, GemvBatch& b, int rows_per_wave)
{
    int order[kGemvMaxLayers];
    for (int l = 0; l < count; l++)
        order[l] = l;
    for (int a = 1; a < count; a++)
        for (int c = a; c > 0 && d[order[c]].K > d[order[c - 1]].K; c--) {
            const int t = order[c];
            order[c] = order[c - 1];
            order[c - 1] = t;
        }
    b = GemvBatch{};
    int nblocks = 0;
    for (int o = 0; o < count; o++) {
        const int l = order[o];
        GemvLayer& L = b.L[b.count++];
        L.q = d[l].q;
        L.s = d[l].s;
        L.z = d[l].z;
        // with no weak columns, point the weak arrays at valid memory (the scales
        // and the first row of x): the kernel reads them unconditionally, ignores them
        L.idx = d[l].k > 0 ? d[l].idx : reinterpret_cast<const int32_t*>(d[l].x);
        L.ww = d[l].k > 0 ? d[l].ww : d[l].s;
        L.x = d[l].x;
        L.y = d[l].y;
        L.N = (int32_t)d[l].N;
        L.K = (int32_t)d[l].K;
        L.k = d[l].k;
        L.block0 = nblocks;
        L.xw = d[l].xw ? d[l].xw : d[l].x;
        L.kw = (int32_t)(d[l].xw ? d[l].kw : d[l].K);
        L.gsh = 0;
        if (groups)
            while ((int64_t)32 << L.gsh < groups[l])
                L.gsh++;
        const int rows = 4 * rows_per_wave;
        nblocks += (int)((d[l].N + rows - 1) / rows);
    }
    return nblocks;
}

}  // namespace

// One launch for the batch; blocks of 4 wavefronts, each wavefront owning
// kRowsPerWave consecutive rows of its layer.
hipError_t launch_gemv(const LinearDesc* d, int count, int M, hipStream_t s)
{
    GemvBatch b;
    int nblocks = build_batch(d, count, nullptr, b, kRowsPerWave);
    const size_t lds = (size_t)M * kChunkTiles * 4 * kQuadStride * 16;
    if (M == 1 && nblocks < kSmallLaunchBlocks && !gemv_products_on_matrix_cores(1)) {
        nblocks = build_batch(d, count, nullptr, b, 2);
        hipLaunchKernelGGL(k_gemv_r2, dim3(nblocks), dim3(256), lds, s, b);
        return hipGetLastError();
    }
    switch (M) {
    case 1: return launch_m<1>(b, nblocks, lds, s);
    case 2: return launch_m<2>(b, nblocks, lds, s);
    case 3: return launch_m<3>(b, nblocks, lds, s);
    default: return launch_m<4>(b, nblocks, lds, s);
    }
}

hipError_t launch_gemv_grouped(const LinearDesc* d, const int64_t* groups, int count, int M, hipStream_t s)
{
    GemvBatch b;
    const int nblocks = build_batch(d, count, groups, b, kRowsPerWave);
    const size_t lds = (size_t)M * kChunkTiles * 4 * kQuadStride * 16;
#define OWQ_GG(MM) hipLaunchKernelGGL((k_gemv_grouped<MM>), dim3(nblocks), dim3(256), lds, s, b)
    switch (M) {
    case 1: OWQ_GG(1); break;
    case 2: OWQ_GG(2); break;
    case 3: OWQ_GG(3); break;
    default: OWQ_GG(4); break;
    }
#undef OWQ_GG
    return hipGetLastError();
}

}  // namespace owq
