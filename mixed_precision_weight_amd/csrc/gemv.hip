// gemv.hip -- decode-time OWQ linear, small batch M (gfx950, vector ALUs).
//
//   y[m][i] = s_i * sum_j (q_ij - z_i) x[m][j] + sum_c w_weak[i][c] x[m][idx_c]
//
// The 3-bit dense matrix is streamed once from HBM; the weak fp16 block is a
// small contiguous [N][k] array and only x is gathered at the weak indices, on
// the fly ([PL] "Real-device acceleration", paper "Acceleration on Real Device"
// p.6; [PL] = paperlayer.ai page "OWQ: Outlier-Aware Weight Quantization for
// Efficient Fine-Tuning and Inference of Large Language Models").
//
// Persistent streaming design. The host gives every layer a number of blocks
// proportional to its bytes; a block of 4 or 8 wavefronts owns a contiguous row
// range of one layer. At block start it stages x (all K, permuted into decode-pair order)
// and the rows' scale, zero point and weak weights in LDS, while each wavefront
// already has a ring of D code tiles in flight. A tile is one 12-byte group per
// lane (64 consecutive groups = 768 contiguous bytes of one row); the wave walks
// its rows (rows rbeg + w, +4, ...) tile by tile, refilling the ring slot it
// just consumed, so loads stay D tiles ahead of the arithmetic and HBM latency
// overlaps the decode of earlier tiles. Rows end in a DPP wave reduction.
//
// Decode without per-code shifts: a 3-bit field that sits inside the mantissa of
// an fp16 half (bits p..p+2 with p <= 7) becomes an exact fp16 number once an
// exponent is OR-ed above it: exponent 2^(10-p) gives the value 2^(10-p) + q.
// With the sequential bit order (code c at bits 3c..3c+2 of the 96-bit group),
// six 32-bit windows of the group (w0>>2, bits 11..42, w1, w1>>9, bits 62..93,
// w2>>7) each hold codes at in-half positions 1/4/7 (low half) and 0/3/6 (high
// half), so one v_and_or_b32 yields a packed pair (off_lo + q_a, off_hi + q_b);
// codes 0 and 31 form the sixteenth pair. One v_pk_add_f16 of the row's
// -(off + z) pair then gives (q_a - z, q_b - z) EXACTLY (small integers), and one
// v_dot2_f32_f16 multiplies it with the matching x pair. Every product is exact,
// so the fp32 sum's error is bounded relative to sum_j |(q_j - z) x_j|, for
// every row, including rows whose codes all equal the zero point. Per tile:
// 5 window ops, 17 and-or, 16 packed subtracts, 16 dot2 per token.
#include <cstdlib>

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
    int32_t block0;    // first block of this layer
    int32_t rpb;       // rows per block
    int32_t ww_vec16;  // w_weak is 16-byte aligned (vector staging)
};

struct GemvBatch {
    GemvLayer L[kGemvMaxLayers];
    int32_t count;
};

// Pair p of a group = (code lo[p], code hi[p]).
__device__ constexpr int kPairLo[16] = {1, 2, 3, 4, 5, 11, 12, 13, 14, 15, 21, 22, 23, 24, 25, 0};
__device__ constexpr int kPairHi[16] = {6, 7, 8, 9, 10, 16, 17, 18, 19, 20, 26, 27, 28, 29, 30, 31};

// Field masks and exponents: low-half positions 1/4/7 with exponents 2^9/2^6/2^3,
// high-half positions 0/3/6 with exponents 2^10/2^7/2^4 -> coefficient 1 on q.
constexpr uint32_t kMaskA = 0x0007000eu, kMagicA = 0x64006000u;  // (512 + q, 1024 + q)
constexpr uint32_t kMaskB = 0x00380070u, kMagicB = 0x58005400u;  // (64 + q, 128 + q)
constexpr uint32_t kMaskC = 0x01c00380u, kMagicC = 0x4c004800u;  // (8 + q, 16 + q)

typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// v_and_or_b32 d = (a & mask) | magic. gfx9 VOP3 takes no literal operands and
// reads at most one SGPR, so the mask goes in an SGPR and the exponent pattern in
// a VGPR; plain C would be split into v_and_b32 + v_or_b32 with two literals.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic)
{
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask), "v"(magic));
    return d;
}

struct Magic {  // exponent patterns held in VGPRs for the whole kernel
    uint32_t a, b, c, p;
};

__device__ __forceinline__ Magic make_magic()
{
    Magic m;
    // opaque to the optimiser so the constants stay in registers
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.a) : "i"(kMagicA));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.b) : "i"(kMagicB));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.c) : "i"(kMagicC));
    asm volatile("v_mov_b32 %0, %1" : "=v"(m.p) : "i"(0x64006400u));
    return m;
}

// -(off + z) for both halves of each pair type, as fp16 bit patterns:
// off + z = 2^E + z has mantissa field z * 2^(10 - E) under exponent E.
struct ZeroSub {
    uint32_t a, b, c, p;
};

__device__ __forceinline__ ZeroSub make_zero_sub(uint32_t z)
{
    ZeroSub n;
    n.a = ((0xe400u | z) << 16) | (0xe000u | (z << 1));          // -(1024 + z), -(512 + z)
    n.b = ((0xd800u | (z << 3)) << 16) | (0xd400u | (z << 4));   // -(128 + z),  -(64 + z)
    n.c = ((0xcc00u | (z << 6)) << 16) | (0xc800u | (z << 7));   // -(16 + z),   -(8 + z)
    n.p = ((0xe400u | z) << 16) | (0xe400u | z);                 // -(1024 + z) twice
    return n;
}

__device__ __forceinline__ uint32_t sub_h2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, as_h2(a) + as_h2(b));
}

// Sixteen exact (q_lo - z, q_hi - z) fp16 pairs of one 96-bit group, in
// kPairLo/kPairHi order.
__device__ __forceinline__ void decode_group(uint32_t w0, uint32_t w1, uint32_t w2, const Magic& mg,
                                             const ZeroSub& n, uint32_t p[16])
{
    const uint32_t a1 = w0 >> 2;
    const uint32_t b1 = __builtin_amdgcn_alignbit(w1, w0, 11);
    const uint32_t a2 = w1;
    const uint32_t b2 = w1 >> 9;
    const uint32_t a3 = __builtin_amdgcn_alignbit(w2, w1, 30);
    const uint32_t b3 = w2 >> 7;
    p[0] = sub_h2(and_or(a1, kMaskA, mg.a), n.a);
    p[1] = sub_h2(and_or(a1, kMaskB, mg.b), n.b);
    p[2] = sub_h2(and_or(a1, kMaskC, mg.c), n.c);
    p[3] = sub_h2(and_or(b1, kMaskA, mg.a), n.a);
    p[4] = sub_h2(and_or(b1, kMaskB, mg.b), n.b);
    p[5] = sub_h2(and_or(a2, kMaskA, mg.a), n.a);
    p[6] = sub_h2(and_or(a2, kMaskB, mg.b), n.b);
    p[7] = sub_h2(and_or(a2, kMaskC, mg.c), n.c);
    p[8] = sub_h2(and_or(b2, kMaskA, mg.a), n.a);
    p[9] = sub_h2(and_or(b2, kMaskB, mg.b), n.b);
    p[10] = sub_h2(and_or(a3, kMaskA, mg.a), n.a);
    p[11] = sub_h2(and_or(a3, kMaskB, mg.b), n.b);
    p[12] = sub_h2(and_or(a3, kMaskC, mg.c), n.c);
    p[13] = sub_h2(and_or(b3, kMaskA, mg.a), n.a);
    p[14] = sub_h2(and_or(b3, kMaskB, mg.b), n.b);
    // (1024 + q0, 1024 + q31): code 0 at bits 0..2 of w0, code 31 at bits 29..31 of w2
    p[15] = sub_h2(and_or(w2 >> 13, 0x00070000u, and_or(w0, 7u, mg.p)), n.p);
}

constexpr int kWeakLds = 256;  // weak columns per row staged in LDS (larger k reads them from HBM)
constexpr int kDepth = 8;      // tiles in flight per wavefront in the generic stream
constexpr int kMaxRowsPerBlock = 256;

// Staged x layout (uint4 units): [m][tile u][quad qd][lane l] for group g = 64 u + l,
// so a lane's four quads of a tile are 1 KB apart (immediate offsets) and the
// lanes of a wave read consecutive 16-byte words.
__device__ __forceinline__ int xs_index(int m, int T, int g) { return ((m * T + (g >> 6)) << 8) + (g & 63); }

__device__ __forceinline__ void store_group(const uint4 (&v)[4], uint4* __restrict__ xs_mg)
{
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        w[4 * i + 0] = v[i].x;
        w[4 * i + 1] = v[i].y;
        w[4 * i + 2] = v[i].z;
        w[4 * i + 3] = v[i].w;
    }
    uint32_t pr[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int lo = kPairLo[i], hi = kPairHi[i];
        uint32_t hl = (w[lo >> 1] >> (16 * (lo & 1))) & 0xffffu;
        uint32_t hh = (w[hi >> 1] >> (16 * (hi & 1))) & 0xffffu;
        pr[i] = hl | (hh << 16);
    }
#pragma unroll
    for (int qd = 0; qd < 4; qd++)
        xs_mg[qd * 64] = make_uint4(pr[4 * qd], pr[4 * qd + 1], pr[4 * qd + 2], pr[4 * qd + 3]);
}

// Byte offset, inside the staged x of token m, of column j (inverse of the pair order).
__device__ __forceinline__ int x_lds_byte(int m, int T, int j)
{
    const int g = j >> 5, c = j & 31;
    int p, h;
    if (c == 0) {
        p = 15;
        h = 0;
    } else if (c == 31) {
        p = 15;
        h = 1;
    } else {
        const int r = (c - 1) / 10, t = (c - 1) - 10 * r;
        h = t >= 5;
        p = 5 * r + (t - 5 * h);
    }
    return ((xs_index(m, T, g) + ((p >> 2) << 6)) << 4) + ((p & 3) << 2) + (h << 1);
}

__host__ __device__ constexpr size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

// LDS layout of a block: x pair quads [M][T][4][64] (uint4); scale [rpb] (fp16); zero
// point [rpb]; row results [M][rpb] (fp32); weak weights [rpb][k] (k <= kWeakLds).
struct GemvLds {
    size_t sc, z, y, ww, total;
    __host__ __device__ GemvLds(int M, int G, int rpb, int k)
    {
        sc = (size_t)M * ((G + 63) / 64) * 64 * 4 * 16;
        z = sc + align16((size_t)rpb * 2);
        y = z + align16((size_t)rpb);
        ww = y + align16((size_t)M * rpb * 4);
        total = ww + (k <= kWeakLds ? align16((size_t)rpb * k * 2) : 0);
    }
};

// ---------------------------------------------------------------- staging --
// Block-level inputs: issued as loads first (registers), committed to LDS after
// the wave's ring of code tiles is in flight, so the staging wait does not queue
// behind the HBM loads of the ring.
constexpr int kWwVec = 4;  // 16-byte weak-weight vectors staged per thread in the first pass

template <int NT>
struct Staging {
    uint4 xa[4];         // one 32-column group of x per thread
    uint4 wv[kWwVec];    // weak weights, 16-byte vectors
    uint16_t sv;         // row scale
    uint8_t zv;          // row zero point
    int wj[4];           // weak indices of this lane
};

struct BlockArgs {
    const uint16_t* X;
    const int32_t* IDX;
    const uint16_t* WW;
    const uint16_t* S;
    const uint8_t* Z;
    int K, G, T, k, rbeg, nrb, rpb;
    bool wl, ww16;
};

template <int M, int NT>
__device__ __forceinline__ void stage_issue(const BlockArgs& a, int tid, int lane, Staging<NT>& st)
{
    const int MG = M * a.G;
    if (tid < MG) {
        const uint4* src = reinterpret_cast<const uint4*>(a.X + (int64_t)(tid / a.G) * a.K + (int64_t)(tid % a.G) * 32);
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
            st.xa[q4] = src[q4];
    }
    st.sv = 0;
    st.zv = 0;
    if (tid < a.nrb) {  // rows per block <= kMaxRowsPerBlock <= threads per block
        st.sv = a.S[a.rbeg + tid];
        st.zv = a.Z[a.rbeg + tid];
    }
    const int E = a.wl ? a.nrb * a.k : 0;
    if (a.ww16) {
        const uint4* src = reinterpret_cast<const uint4*>(a.WW + (int64_t)a.rbeg * a.k);
#pragma unroll
        for (int t = 0; t < kWwVec; t++) {
            const int i = tid + NT * t;
            st.wv[t] = (8 * i < E) ? src[i] : make_uint4(0, 0, 0, 0);
        }
    }
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int c = lane + 64 * v;
        const int j = c < a.k ? a.IDX[c] : 0;
        st.wj[v] = (j >= 0 && j < a.K) ? j : 0;
    }
}

// LDS writes of the staged inputs, the block barrier, then this lane's x values at
// the weak indices (read back from the staged x).
template <int M, int NT>
__device__ __forceinline__ void stage_commit(const BlockArgs& a, int tid, int lane, const Staging<NT>& st, char* base,
                                             uint4* xs, uint16_t* s_sc, uint8_t* s_z, uint16_t* s_ww,
                                             float (&xw)[M][4])
{
    const int MG = M * a.G;
    if (tid < MG)
        store_group(st.xa, xs + xs_index(tid / a.G, a.T, tid % a.G));
    for (int i = tid + NT; i < MG; i += NT) {  // M * G > threads: direct copies
        const uint4* src = reinterpret_cast<const uint4*>(a.X + (int64_t)(i / a.G) * a.K + (int64_t)(i % a.G) * 32);
        uint4 v[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)
            v[q4] = src[q4];
        store_group(v, xs + xs_index(i / a.G, a.T, i % a.G));
    }
    if (tid < a.nrb) {
        s_sc[tid] = st.sv;
        s_z[tid] = st.zv;
    }
    const int E = a.wl ? a.nrb * a.k : 0;
    if (a.ww16) {
        uint4* dst = reinterpret_cast<uint4*>(s_ww);
#pragma unroll
        for (int t = 0; t < kWwVec; t++) {
            const int i = tid + NT * t;
            if (8 * i < E)
                dst[i] = st.wv[t];
        }
        const uint4* src = reinterpret_cast<const uint4*>(a.WW + (int64_t)a.rbeg * a.k);
        for (int i = tid + kWwVec * NT; 8 * i < E; i += NT)
            dst[i] = src[i];
    } else {
        for (int i = tid; i < E; i += NT)
            s_ww[i] = a.WW[(int64_t)a.rbeg * a.k + i];
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < 4; v++) {
        const int c = lane + 64 * v;
#pragma unroll
        for (int m = 0; m < M; m++)
            xw[m][v] = c < a.k ? h2f(*reinterpret_cast<const uint16_t*>(base + x_lds_byte(m, a.T, st.wj[v]))) : 0.0f;
    }
}

// ------------------------------------------------------------ row context --
template <int M>
struct RowCtx {
    Magic mg;
    const uint4* xs;
    const uint16_t* s_sc;
    const uint8_t* s_z;
    float* s_y;
    const uint16_t* s_ww;
    int rpb, T, G, k;
    bool wl;
    int lane;
};

// Row start: zero-point constants and scale of block row rl (LDS).
template <int M>
__device__ __forceinline__ void row_begin(const RowCtx<M>& cx, int rl, ZeroSub& nz, float& sc, float (&acc)[M])
{
    const uint32_t z = (uint32_t)__builtin_amdgcn_readfirstlane((int)cx.s_z[rl]);
    nz = make_zero_sub(z);
    sc = h2f(cx.s_sc[rl]);
#pragma unroll
    for (int m = 0; m < M; m++)
        acc[m] = 0.0f;
}

// One tile (group g of every token) of the current row.
template <int M>
__device__ __forceinline__ void tile_dot(const RowCtx<M>& cx, const u32x3& w, int g, const ZeroSub& nz,
                                         float (&acc)[M])
{
    uint32_t p[16];
    decode_group(w.x, w.y, w.z, cx.mg, nz, p);
#pragma unroll
    for (int m = 0; m < M; m++) {
        float a = acc[m];
        const uint4* xq4 = cx.xs + xs_index(m, cx.T, g);
#pragma unroll
        for (int qd = 0; qd < 4; qd++) {
            const uint4 xq = xq4[qd << 6];
            a = dot2(p[4 * qd + 0], xq.x, a);
            a = dot2(p[4 * qd + 1], xq.y, a);
            a = dot2(p[4 * qd + 2], xq.z, a);
            a = dot2(p[4 * qd + 3], xq.w, a);
        }
        acc[m] = a;
    }
}

// Per-lane partial of a finished row: scale times the dense dot, plus this
// lane's share of the weak columns (staged in LDS).
template <int M>
__device__ __forceinline__ void row_partial(const RowCtx<M>& cx, int rl, float sc, const float (&acc)[M],
                                            const float (&xw)[M][4], float (&part)[M])
{
#pragma unroll
    for (int m = 0; m < M; m++)
        part[m] = sc * acc[m];
    if (cx.wl) {
#pragma unroll
        for (int v = 0; v < 4; v++) {
            const int c = cx.lane + 64 * v;
            if (c < cx.k) {
                const float w = h2f(cx.s_ww[rl * cx.k + c]);
#pragma unroll
                for (int m = 0; m < M; m++)
                    part[m] += w * xw[m][v];
            }
        }
    }
}

__device__ __forceinline__ float f_of(uint32_t v) { return __builtin_bit_cast(float, v); }
__device__ __forceinline__ uint32_t u_of(float v) { return __builtin_bit_cast(uint32_t, v); }

// Sum over the 64 lanes of R per-lane values at once (R = 4, 8 or 16): lane-half
// swaps (v_permlane32_swap, then v_permlane16_swap) each add two values while
// halving their lane span, then a DPP reduction inside 16-lane rows. On return,
// value v holds, in lanes 16 q .. 16 q + 15, the total of input R / 4 * q + v.
template <int R>
__device__ __forceinline__ void reduce_rows(float (&a)[R])
{
    static_assert(R == 4 || R == 8 || R == 16, "R");
    constexpr int H = R / 2, Q = R / 4;
    float b[H];
#pragma unroll
    for (int i = 0; i < H; i++) {  // pairs (i, i + H): lanes 0-31 keep input i, 32-63 input i + H
        auto t = __builtin_amdgcn_permlane32_swap(u_of(a[i]), u_of(a[i + H]), false, false);
        b[i] = f_of(t[0]) + f_of(t[1]);
    }
#pragma unroll
    for (int i = 0; i < Q; i++) {  // pairs (i, i + Q) inside each half
        auto t = __builtin_amdgcn_permlane16_swap(u_of(b[i]), u_of(b[i + Q]), false, false);
        a[i] = f_of(t[0]) + f_of(t[1]);
    }
#pragma unroll
    for (int i = 0; i < Q; i++) {
        float v = a[i];
        v += dpp_f<0xb1>(v);   // quad_perm [1,0,3,2]
        v += dpp_f<0x4e>(v);   // quad_perm [2,3,0,1]
        v += dpp_f<0x124>(v);  // row_ror:4
        v += dpp_f<0x128>(v);  // row_ror:8
        a[i] = v;
    }
}
// After reduce_rows<R>, input r = i + Q * ((lane >> 4) ...) : lanes 16q..16q+15 of
// a[i] hold input index i + (q & 1) * H ... see row_of().
template <int R>
__device__ __forceinline__ int reduced_index(int i, int q)
{
    // quarter q: half h = q >> 1 selects +H (step 1), odd quarter selects +Q (step 2)
    return i + (q & 1) * (R / 4) + (q >> 1) * (R / 2);
}

// Stream for rows of exactly T tiles. The ring holds RPR whole rows (T * RPR
// tiles); a tile's offset inside its row is an instruction immediate and the row
// offset a scalar, so the loop carries no per-tile bookkeeping. Every RPR rows
// the per-lane partials are reduced together (reduce_rows).
template <int M, int T, int RPR, int WAVES, int NT>
__device__ __forceinline__ void stream_rows(const RowCtx<M>& cx, const BlockArgs& ba, const Staging<NT>& st, char* base,
                                            uint4* xs, uint16_t* s_sc, uint8_t* s_z, uint16_t* s_ww,
                                            __amdgpu_buffer_rsrc_t qr, int voff, int wave, int nrw, int tid)
{
    const int rstride = WAVES * cx.G * 12;
    u32x3 cw[RPR][T];
    int pre = wave * cx.G * 12;  // byte offset of the next row to prefetch
#pragma unroll
    for (int rr = 0; rr < RPR; rr++) {
        const int so = rr < nrw ? pre : 0x7ffff000;
#pragma unroll
        for (int u = 0; u < T; u++)
            cw[rr][u] = __builtin_amdgcn_raw_buffer_load_b96(qr, voff + u * 768, so, 0);
        pre += rstride;
    }
    float xw[M][4];
    stage_commit<M, NT>(ba, tid, cx.lane, st, base, xs, s_sc, s_z, s_ww, xw);

    constexpr int RR = RPR < 4 ? 4 : RPR;  // rows per reduction (zero-padded)
    ZeroSub nz = make_zero_sub(0);
    float sc = 0.0f;
    for (int j0 = 0; j0 < nrw; j0 += RPR) {
        float part[M][RR];
#pragma unroll
        for (int rr = 0; rr < RR; rr++)
#pragma unroll
            for (int m = 0; m < M; m++)
                part[m][rr] = 0.0f;
#pragma unroll
        for (int rr = 0; rr < RPR; rr++) {
            const int j = j0 + rr;
            if (j < nrw) {
                const int rl = wave + WAVES * j;
                float acc[M];
                row_begin(cx, rl, nz, sc, acc);
#pragma unroll
                for (int u = 0; u < T; u++) {
                    const int g = (u << 6) + cx.lane;
                    if (u < T - 1 || g < cx.G)
                        tile_dot(cx, cw[rr][u], g, nz, acc);
                }
                float pt[M];
                row_partial(cx, rl, sc, acc, xw, pt);
#pragma unroll
                for (int m = 0; m < M; m++)
                    part[m][rr] = pt[m];
            }
            const int so = j + RPR < nrw ? pre : 0x7ffff000;
#pragma unroll
            for (int u = 0; u < T; u++)
                cw[rr][u] = __builtin_amdgcn_raw_buffer_load_b96(qr, voff + u * 768, so, 0);
            pre += rstride;
        }
        const int q = cx.lane >> 4;
#pragma unroll
        for (int m = 0; m < M; m++) {
            reduce_rows<RR>(part[m]);
#pragma unroll
            for (int i = 0; i < RR / 4; i++) {
                const int rr = reduced_index<RR>(i, q);
                const int j = j0 + rr;
                if ((cx.lane & 15) == 0 && rr < RPR && j < nrw)
                    cx.s_y[m * cx.rpb + wave + WAVES * j] = part[m][i];
            }
        }
    }
}

// Generic stream (any tiles per row): a ring of D tiles walked tile by tile,
// one 64-lane reduction per row.
template <int M, int D, int WAVES, int NT>
__device__ __forceinline__ void stream_tiles(const RowCtx<M>& cx, const BlockArgs& ba, const Staging<NT>& st, char* base,
                                             uint4* xs, uint16_t* s_sc, uint8_t* s_z, uint16_t* s_ww,
                                             __amdgpu_buffer_rsrc_t qr, int voff, int wave, int nrw, int tid)
{
    const int T = cx.T;
    const int total = nrw * T;
    const int rstride = WAVES * cx.G * 12;
    int prow = wave * cx.G * 12;
    int pu = 0, pj = 0;
    u32x3 cw[D];
#pragma unroll
    for (int d = 0; d < D; d++) {
        const int so = pj < nrw ? prow + pu * 768 : 0x7ffff000;
        cw[d] = __builtin_amdgcn_raw_buffer_load_b96(qr, voff, so, 0);
        if (++pu == T) {
            pu = 0;
            ++pj;
            prow += rstride;
        }
    }
    float xw[M][4];
    stage_commit<M, NT>(ba, tid, cx.lane, st, base, xs, s_sc, s_z, s_ww, xw);

    ZeroSub nz = make_zero_sub(0);
    float sc = 0.0f;
    float acc[M];
    int cj = 0, cu = 0;
    for (int f0 = 0; f0 < total; f0 += D) {
#pragma unroll
        for (int d = 0; d < D; d++) {
            if (f0 + d < total) {
                const int rl = wave + WAVES * cj;
                if (cu == 0)
                    row_begin(cx, rl, nz, sc, acc);
                const int g = (cu << 6) + cx.lane;
                if (g < cx.G)
                    tile_dot(cx, cw[d], g, nz, acc);
                if (cu == T - 1) {
                    float pt[M];
                    row_partial(cx, rl, sc, acc, xw, pt);
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        const float t = wave_sum_dpp(pt[m]);
                        if (cx.lane == 0)
                            cx.s_y[m * cx.rpb + rl] = t;
                    }
                    cu = 0;
                    ++cj;
                } else {
                    ++cu;
                }
            }
            const int so = pj < nrw ? prow + pu * 768 : 0x7ffff000;
            cw[d] = __builtin_amdgcn_raw_buffer_load_b96(qr, voff, so, 0);
            if (++pu == T) {
                pu = 0;
                ++pj;
                prow += rstride;
            }
        }
    }
}

// Row-shape class of a layer: its tiles per row when a specialised stream exists
// (1, 2, 3, 4 or 6), else 0 (generic tile stream).
__host__ __device__ constexpr int row_class(int T) { return (T >= 1 && T <= 4) || T == 6 ? T : 0; }
__host__ __device__ constexpr int rows_per_ring(int TC) { return TC == 1 ? 8 : TC == 2 ? 4 : TC == 3 ? 4 : 2; }

template <int M, int TC, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(GemvBatch b)
{
    constexpr int NT = 64 * WAVES;  // threads per block
    static_assert(NT >= kMaxRowsPerBlock, "one staging pass per row");
    extern __shared__ uint4 smem[];
    int li = 0;
    for (int l = 1; l < b.count; l++)
        if ((int)blockIdx.x >= b.L[l].block0)
            li = l;
    BlockArgs ba;
    ba.X = b.L[li].x;
    ba.IDX = b.L[li].idx;
    ba.WW = b.L[li].ww;
    ba.S = b.L[li].s;
    ba.Z = b.L[li].z;
    ba.K = b.L[li].K;
    ba.G = ba.K >> 5;
    ba.T = (ba.G + 63) >> 6;
    ba.k = b.L[li].k;
    ba.rpb = b.L[li].rpb;
    ba.rbeg = ((int)blockIdx.x - b.L[li].block0) * ba.rpb;
    const int N = b.L[li].N;
    ba.nrb = min(N - ba.rbeg, ba.rpb);
    ba.wl = ba.k <= kWeakLds;
    ba.ww16 = b.L[li].ww_vec16;
    const int tid = threadIdx.x, lane = tid & 63;
    // wave-uniform (the compiler cannot infer it from threadIdx.x >> 6)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const GemvLds lay(M, ba.G, ba.rpb, ba.k);
    char* base = reinterpret_cast<char*>(smem);
    uint4* xs = smem;
    uint16_t* s_sc = reinterpret_cast<uint16_t*>(base + lay.sc);
    uint8_t* s_z = reinterpret_cast<uint8_t*>(base + lay.z);
    float* s_y = reinterpret_cast<float*>(base + lay.y);
    uint16_t* s_ww = reinterpret_cast<uint16_t*>(base + lay.ww);

    Staging<NT> st;
    stage_issue<M, NT>(ba, tid, lane, st);

    // this wave's rows: rbeg + wave + WAVES * j, j < nrw; code tiles are raw buffer
    // loads over the block's rows (a per-lane offset lane * 12 plus a wave-uniform
    // scalar offset); lanes past a row's last group read neighbouring codes that
    // are never used, offsets past the block's range read 0
    const __amdgpu_buffer_rsrc_t qr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint32_t*>(b.L[li].q) + (int64_t)ba.rbeg * ba.G * 3, (short)0, ba.nrb * ba.G * 12, 0x00020000);
    const int nrw = ba.nrb - wave > 0 ? (ba.nrb - wave + WAVES - 1) / WAVES : 0;
    const int voff = lane * 12;

    const Magic mg = make_magic();
    RowCtx<M> cx{mg, xs, s_sc, s_z, s_y, s_ww, ba.rpb, ba.T, ba.G, ba.k, ba.wl, lane};
    if constexpr (TC == 0)
        stream_tiles<M, kDepth, WAVES, NT>(cx, ba, st, base, xs, s_sc, s_z, s_ww, qr, voff, wave, nrw, tid);
    else
        stream_rows<M, TC, rows_per_ring(TC), WAVES, NT>(cx, ba, st, base, xs, s_sc, s_z, s_ww, qr, voff, wave, nrw,
                                                         tid);

    // k > kWeakLds: weak columns straight from HBM, after the stream
    if (!ba.wl) {
        for (int j = 0; j < nrw; j++) {
            const int rl = wave + WAVES * j;
            float part[M];
#pragma unroll
            for (int m = 0; m < M; m++)
                part[m] = 0.0f;
            for (int c = lane; c < ba.k; c += 64) {
                int jj = ba.IDX[c];
                jj = (jj >= 0 && jj < ba.K) ? jj : 0;
                const float w = h2f(ba.WW[(int64_t)(ba.rbeg + rl) * ba.k + c]);
#pragma unroll
                for (int m = 0; m < M; m++)
                    part[m] += w * h2f(ba.X[(int64_t)m * ba.K + jj]);
            }
#pragma unroll
            for (int m = 0; m < M; m++) {
                const float t = wave_sum_dpp(part[m]);
                if (lane == 0)
                    s_y[m * ba.rpb + rl] += t;
            }
        }
    }
    __syncthreads();
    uint16_t* __restrict__ Y = b.L[li].y;
    for (int i = tid; i < M * ba.nrb; i += NT) {
        const int m = i / ba.nrb, r = i - m * ba.nrb;
        Y[(int64_t)m * N + ba.rbeg + r] = f2h(s_y[m * ba.rpb + r]);
    }
}

constexpr int kWaves = 8;  // wavefronts per block

template <int M, int TC>
hipError_t launch_mc(const GemvBatch& b, int nblocks, size_t lds, hipStream_t s)
{
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv<M, TC, kWaves>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess)
            return e;
        attr_set = true;
    }
    hipLaunchKernelGGL((k_gemv<M, TC, kWaves>), dim3(nblocks), dim3(64 * kWaves), lds, s, b);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const GemvBatch& b, int tc, int nblocks, size_t lds, hipStream_t s)
{
    if constexpr (M == 1) {
        switch (tc) {
        case 1: return launch_mc<M, 1>(b, nblocks, lds, s);
        case 2: return launch_mc<M, 2>(b, nblocks, lds, s);
        case 3: return launch_mc<M, 3>(b, nblocks, lds, s);
        case 4: return launch_mc<M, 4>(b, nblocks, lds, s);
        case 6: return launch_mc<M, 6>(b, nblocks, lds, s);
        default: break;
        }
    } else if constexpr (M == 2) {
        switch (tc) {
        case 1: return launch_mc<M, 1>(b, nblocks, lds, s);
        case 2: return launch_mc<M, 2>(b, nblocks, lds, s);
        default: break;
        }
    }
    return launch_mc<M, 0>(b, nblocks, lds, s);
}

int target_blocks()
{
    static const int t = [] {
        const char* e = getenv("OWQ_GEMV_BLOCKS");
        int v = e ? atoi(e) : 0;
        return v > 0 ? v : 512;
    }();
    return t;
}

}  // namespace

int gemv_max_tokens(int64_t K)
{
    // x of all tokens lives in LDS: M * K * 2 bytes, kept to 64 KB (128 KB for M = 1)
    int64_t m = 32768 / K;
    if (m > kGemvMaxM)
        m = kGemvMaxM;
    return m < 1 ? 1 : (int)m;
}

bool gemv_fits(int64_t M, int64_t K)
{
    // x (M * K * 2) plus at most 16 KB of staged row data within the 160 KB of LDS
    return M >= 1 && M <= kGemvMaxM && M * K * 2 + 16384 + 64 <= 160 * 1024;
}

// One launch per row-shape class present in the batch (layers of one class share
// a specialised kernel); blocks per layer are proportional to the layer's bytes.
hipError_t launch_gemv(const LinearDesc* d, int count, int M, hipStream_t s)
{
    const int target = target_blocks();
    const int classes[6] = {1, 2, 3, 4, 6, 0};
    auto class_of = [M](int64_t K) {
        const int T = (int)((K / 32 + 63) / 64);
        return M == 1 ? row_class(T) : (M == 2 && T <= 2 ? T : 0);
    };
    for (int ci = 0; ci < 6; ci++) {
        const int tc = classes[ci];
        double total = 0.0;  // bytes of this class: each launch spreads over the whole GPU
        for (int l = 0; l < count; l++)
            if (class_of(d[l].K) == tc)
                total += (double)d[l].N * (double)d[l].K;
        GemvBatch b{};
        int nblocks = 0;
        size_t lds = 0;
        for (int l = 0; l < count; l++) {
            const int G = (int)(d[l].K / 32);
            if (class_of(d[l].K) != tc)
                continue;
            GemvLayer& L = b.L[b.count++];
            L.q = d[l].q;
            L.s = d[l].s;
            L.z = d[l].z;
            L.idx = d[l].idx;
            L.ww = d[l].ww;
            L.x = d[l].x;
            L.y = d[l].y;
            L.N = (int32_t)d[l].N;
            L.K = (int32_t)d[l].K;
            L.k = d[l].k;
            L.ww_vec16 = d[l].k > 0 && ((uintptr_t)d[l].ww % 16) == 0 ? 1 : 0;
            int nb = (int)((double)target * (double)d[l].N * (double)d[l].K / total + 0.5);
            nb = nb < 1 ? 1 : nb;
            int rpb = (int)((d[l].N + nb - 1) / nb);
            rpb = (rpb + 7) & ~7;  // rows for every wave; 16-byte aligned weak-weight rows
            // per-block row data in LDS kept to ~16 KB
            const int rowbytes = 3 + 4 * M + (d[l].k <= kWeakLds ? 2 * d[l].k : 0);
            int cap = (16384 / rowbytes) & ~7;
            cap = cap < 8 ? 8 : cap;
            cap = cap > kMaxRowsPerBlock ? kMaxRowsPerBlock : cap;
            rpb = rpb < cap ? rpb : cap;
            L.rpb = rpb;
            L.block0 = nblocks;
            nblocks += (int)((d[l].N + rpb - 1) / rpb);
            const size_t ll = GemvLds(M, G, rpb, d[l].k).total;
            lds = ll > lds ? ll : lds;
        }
        if (b.count == 0)
            continue;
        hipError_t e;
        switch (M) {
        case 1: e = launch_m<1>(b, tc, nblocks, lds, s); break;
        case 2: e = launch_m<2>(b, tc, nblocks, lds, s); break;
        case 3: e = launch_m<3>(b, tc, nblocks, lds, s); break;
        default: e = launch_m<4>(b, tc, nblocks, lds, s); break;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace owq
