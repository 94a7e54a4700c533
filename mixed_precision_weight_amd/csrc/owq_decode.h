// owq_decode.h -- register decode of the packed 3-bit groups (gfx950), shared
// by the vector-ALU and the matrix-core linear kernels.
//
// A group holds the 32 codes of one row's 32 columns in the 96-bit word
// w0 | w1 << 32 | w2 << 64, as 32 three-bit slots (slot s at bits 3s..3s+2);
// columns 2p and 2p + 1 sit in slots kPairLo[p] and kPairHi[p]. A 3-bit field
// that sits inside the mantissa of an fp16 half (bits p..p+2 with p <= 7)
// becomes an exact fp16 number once an exponent is OR-ed above it: exponent
// 2^(10-p) gives the value 2^(10-p) + q. Six 32-bit windows of the group (w0>>2,
// bits 11..42, w1, w1>>9, bits 62..93, w2>>7) each hold slots at in-half
// positions 1/4/7 (low half) and 0/3/6 (high half), so one v_and_or_b32 yields a
// packed pair (off_lo + q_a, off_hi + q_b); slots 0 and 31 form the sixteenth
// pair. One v_pk_add_f16 of the row's -(off + z) pair then gives
// (q_a - z, q_b - z) EXACTLY (small integers). Because of the slot layout, decode
// pair p is columns (2p, 2p + 1): the sixteen pairs come out in natural column
// order and meet x as it is stored, one dword per column pair.
#pragma once

#include "owq_device.h"

namespace owq {
namespace {

// Decode pair p = the slots (kPairLo[p], kPairHi[p]) = columns (2p, 2p + 1).
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

// The four pairs 4 qd .. 4 qd + 3 of a group (columns 8 qd .. 8 qd + 7), the same
// values as decode_group's p[4 qd .. 4 qd + 3].
template <int QD>
__device__ __forceinline__ void decode_quad(uint32_t w0, uint32_t w1, uint32_t w2, const Magic& mg,
                                            const ZeroSub& n, uint32_t p[4])
{
    if constexpr (QD == 0) {
        const uint32_t a1 = w0 >> 2;
        p[0] = sub_h2(and_or(a1, kMaskA, mg.a), n.a);
        p[1] = sub_h2(and_or(a1, kMaskB, mg.b), n.b);
        p[2] = sub_h2(and_or(a1, kMaskC, mg.c), n.c);
        p[3] = sub_h2(and_or(__builtin_amdgcn_alignbit(w1, w0, 11), kMaskA, mg.a), n.a);
    } else if constexpr (QD == 1) {
        p[0] = sub_h2(and_or(__builtin_amdgcn_alignbit(w1, w0, 11), kMaskB, mg.b), n.b);
        p[1] = sub_h2(and_or(w1, kMaskA, mg.a), n.a);
        p[2] = sub_h2(and_or(w1, kMaskB, mg.b), n.b);
        p[3] = sub_h2(and_or(w1, kMaskC, mg.c), n.c);
    } else if constexpr (QD == 2) {
        const uint32_t b2 = w1 >> 9;
        const uint32_t a3 = __builtin_amdgcn_alignbit(w2, w1, 30);
        p[0] = sub_h2(and_or(b2, kMaskA, mg.a), n.a);
        p[1] = sub_h2(and_or(b2, kMaskB, mg.b), n.b);
        p[2] = sub_h2(and_or(a3, kMaskA, mg.a), n.a);
        p[3] = sub_h2(and_or(a3, kMaskB, mg.b), n.b);
    } else {
        const uint32_t b3 = w2 >> 7;
        p[0] = sub_h2(and_or(__builtin_amdgcn_alignbit(w2, w1, 30), kMaskC, mg.c), n.c);
        p[1] = sub_h2(and_or(b3, kMaskA, mg.a), n.a);
        p[2] = sub_h2(and_or(b3, kMaskB, mg.b), n.b);
        p[3] = sub_h2(and_or(w2 >> 13, 0x00070000u, and_or(w0, 7u, mg.p)), n.p);
    }
}

}  // namespace
}  // namespace owq
