// owq_device.h -- device helpers shared by the gfx950 kernels of libowq.
//
// fp16 values travel as IEEE binary16 bit patterns (uint16_t). Conversions use
// the hardware's round-to-nearest-even (v_cvt_f16_f32) and exact widening.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace owq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float h2f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// ---------------------------------------------------------------- quantiser --
// Min-max round-to-nearest on a 3-bit asymmetric grid (7 steps). The range
// [lo, hi] always contains 0. Step: fp32 (hi - lo) / 7, IEEE division, rounded
// once to fp16; zero point: rint(-lo / step) clamped to [0, 7]; a row with
// hi == lo, or whose step rounds to fp16 zero, uses step 1 and zero point 0.
// code(w) = clamp(rint(w / step) + z, 0, 7) with rint = round half to even.
// These are the same IEEE operations, in the same order, as the definition;
// the translation units that call them are compiled without FMA contraction.
__device__ __forceinline__ void qparams_from_range(float lo, float hi, uint16_t& s16, int& z)
{
    if (hi == lo) {
        s16 = 0x3c00;
        z = 0;
        return;
    }
    float s32 = (hi - lo) / 7.0f;
    uint16_t s = f2h(s32);
    if ((s & 0x7fff) == 0) {
        s16 = 0x3c00;
        z = 0;
        return;
    }
    float sf = h2f(s);
    float zr = rintf(-lo / sf);
    z = zr < 0.0f ? 0 : (zr > 7.0f ? 7 : (int)zr);
    s16 = s;
}

// Per-row constants of the round-to-nearest step for a positive fp16 step s
// and zero point z.
struct RtnRow {
    float s;       // step
    float rs;      // ~1/s (hardware reciprocal, within a few ulps)
    float hs;      // s / 2
    float tie;     // 2^14 rs: scales the distance to s / 2, see rint_quotient
    float lo, hi;  // -z and 7 - z: the range of code - z
    float zf;      // z
};

__device__ __forceinline__ RtnRow make_rtn_row(float s, int z)
{
    const float rs = __builtin_amdgcn_rcpf(s);
    return RtnRow{s, rs, 0.5f * s, 16384.0f * rs, -(float)z, 7.0f - (float)z, (float)z};
}

// rint(w / s), round half to even, for an fp16 weight w, with neither an IEEE
// division nor a compare. The guess t = rint(w rs) differs from w / s by at
// most 4e-6 for |w / s| <= 16, and a quotient of two fp16 values is either a
// half-integer or at least 2^-13 away from one (its distance to h + 1/2 is a
// multiple of an ulp of w or s over 2s). So t is the nearest integer, and
// e = w - t s (exact after one FMA: t s has at most 16 significant bits) has
// |e| < s / 2, except at an exact half-integer, where |e| = s / 2 and t may be
// the odd neighbour. d = s / 2 - |e| is then 0, and at least s 2^-13 in every
// other case, so f = max(1/2 - 2^14 d / s, 0) is 1/2 at a tie and 0 otherwise,
// and rint(t + copysign(f, e)) takes a tie to the even neighbour. The guess is
// clamped to +-16; beyond that (where |e| may exceed s / 2 and f 1/2) only the
// side matters to the callers' clamp.
__device__ __forceinline__ float rint_quotient(float w, const RtnRow& r)
{
    const float t = __builtin_amdgcn_fmed3f(rintf(w * r.rs), -16.0f, 16.0f);
    const float e = __builtin_fmaf(-t, r.s, w);
    const float d = r.hs - fabsf(e);
    const float f = fmaxf(__builtin_fmaf(-d, r.tie, 0.5f), 0.0f);
    return rintf(t + __builtin_copysignf(f, e));
}

// Grid offset of w: clamp(rint(w / s) + z, 0, 7) - z, as a float.
__device__ __forceinline__ float grid_offset(float w, const RtnRow& r)
{
    return __builtin_amdgcn_fmed3f(rint_quotient(w, r), r.lo, r.hi);
}

// The 3-bit code of w.
__device__ __forceinline__ int rtn_code(float w, const RtnRow& r)
{
    return (int)(grid_offset(w, r) + r.zf);
}

// ---------------------------------------------------------- wave reductions --
// Butterfly over the 64 lanes of a wavefront (deterministic order; every lane
// ends with the full result).
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ float wave_min(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fminf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// DPP butterfly sum over 64 lanes: quad swaps and row rotations reduce each
// 16-lane row, row broadcasts fold the rows into lane 63, which is returned
// (as a wave-uniform value). No LDS traffic, ~7 dependent VALU steps.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_f(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS,
                                                                0xf, false));
}

__device__ __forceinline__ float wave_sum_dpp(float v)
{
    v += dpp_f<0xb1>(v);        // quad_perm [1,0,3,2]
    v += dpp_f<0x4e>(v);        // quad_perm [2,3,0,1]
    v += dpp_f<0x124>(v);       // row_ror:4
    v += dpp_f<0x128>(v);       // row_ror:8  -> every lane holds its 16-lane row sum
    v += dpp_f<0x142, 0xa>(v);  // row_bcast:15 into rows 1, 3
    v += dpp_f<0x143, 0xc>(v);  // row_bcast:31 into rows 2, 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// The same DPP pattern for min / max: lanes a row mask leaves out keep their own
// value. Both are exact, so the order of the steps does not matter.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ float dpp_keep(float v)
{
    const int b = __builtin_bit_cast(int, v);
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, ROWS, 0xf, false));
}

__device__ __forceinline__ float wave_min_dpp(float v)
{
    v = fminf(v, dpp_keep<0xb1>(v));
    v = fminf(v, dpp_keep<0x4e>(v));
    v = fminf(v, dpp_keep<0x124>(v));
    v = fminf(v, dpp_keep<0x128>(v));
    v = fminf(v, dpp_keep<0x142, 0xa>(v));
    v = fminf(v, dpp_keep<0x143, 0xc>(v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max_dpp(float v)
{
    v = fmaxf(v, dpp_keep<0xb1>(v));
    v = fmaxf(v, dpp_keep<0x4e>(v));
    v = fmaxf(v, dpp_keep<0x124>(v));
    v = fmaxf(v, dpp_keep<0x128>(v));
    v = fmaxf(v, dpp_keep<0x142, 0xa>(v));
    v = fmaxf(v, dpp_keep<0x143, 0xc>(v));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ double shfl_xor_f64(double v, int o)
{
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
    lo = __shfl_xor(lo, o, 64);
    hi = __shfl_xor(hi, o, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

}  // namespace owq
