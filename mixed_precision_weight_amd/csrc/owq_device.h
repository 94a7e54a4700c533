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

// rint(w / s), round half to even, for a positive fp16 step s and an fp16 weight
// w, with neither an IEEE division nor a branch (rs ~ 1/s, within a few ulps,
// hs = s / 2). The guess t = rint(w rs) is at most one off, and only when w / s
// lies within a few ulps of a half-integer. e = w - t s is exact after one FMA
// (t s has at most 16 significant bits and e stays within a step of 0), so |e|
// against s/2 classifies the quotient t + e/s exactly: below, t; above, t + 1
// toward e; equal, the exact half-integer t +- 1/2, which rint takes to the even
// neighbour. The quotient of two fp16 values is never within half an fp32 ulp
// of a half-integer without being equal to it, so the result equals rint of the
// correctly rounded fp32 quotient, as in the definition. The guess is clamped
// to +-16; beyond that only the side matters to the callers' clamp.
__device__ __forceinline__ float rint_quotient(float w, float s, float rs, float hs)
{
    const float t = fminf(fmaxf(rintf(w * rs), -16.0f), 16.0f);
    const float e = __builtin_fmaf(-t, s, w);
    const float a = fabsf(e);
    const float f = a > hs ? 1.0f : (a == hs ? 0.5f : 0.0f);
    return rintf(t + __builtin_copysignf(f, e));
}

// Grid offset of w: clamp(rint(w / s) + z, 0, 7) - z, as a float (rs ~ 1/s,
// hs = s / 2, zf = z).
__device__ __forceinline__ float grid_offset(float w, float s, float rs, float hs, float zf)
{
    return fminf(fmaxf(rint_quotient(w, s, rs, hs) + zf, 0.0f), 7.0f) - zf;
}

// The 3-bit code of w.
__device__ __forceinline__ int rtn_code(float w, float s, float rs, float hs, float zf)
{
    return (int)(grid_offset(w, s, rs, hs, zf) + zf);
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

__device__ __forceinline__ double shfl_xor_f64(double v, int o)
{
    uint64_t b = __builtin_bit_cast(uint64_t, v);
    uint32_t lo = (uint32_t)b, hi = (uint32_t)(b >> 32);
    lo = __shfl_xor(lo, o, 64);
    hi = __shfl_xor(hi, o, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

}  // namespace owq
