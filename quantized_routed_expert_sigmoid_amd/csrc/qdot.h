/*
 * qdot.h -- unpacking of the quantised weight containers and the exact int32
 * block partial of the integer dot path.
 *
 * Container layouts ("colibrì 深度拆解", section 5.1, for int4; int2 by the same
 * most-significant-first rule; the README translation "Show HN: 如何在我的低配置
 * 电脑上运行 GLM-5.2", quantised-kernel item: packed layouts equal the int8
 * container bit for bit).  A 32-element block occupies BITS 32-bit words.
 *
 * No element is ever sign-extended on its own.  Each packed field is instead
 * shifted to the top of its byte, which is then the two's-complement int8
 * value (2^(8-BITS)) * v; the byte dot products of v_dot4_i32_i8 are summed
 * exactly and the block total is shifted back right by (8 - BITS), which is
 * exact because every term is a multiple of 2^(8-BITS).  The activation codes
 * are permuted once per block so that their byte order matches the order in
 * which the fields come out of the words.
 *
 * The VALU kernels take int4 another way (prep_dot / block_dot): the
 * weight nibbles are used in place by v_dot8_i32_i4, against two nibble
 * planes of the activation codes.  Every int8 code splits exactly as
 * x = 16 h + l + 8 with h = x >> 4 and l = (x & 15) - 8, both in [-8, 7], so
 * the block dot is 16 sum(q h) + sum(q l) + 8 sum(q): three dot8 per weight
 * word and no unpacking.
 *
 * The file is included by the gfx950 kernels, which define COLI_PERM as
 * __builtin_amdgcn_perm, COLI_SDOT4 as __builtin_amdgcn_sdot4 and COLI_SDOT8
 * as __builtin_amdgcn_sdot8, and by a CPU harness (tests) that defines them
 * as emulations to check the layout logic against direct sums.
 * It needs COLI_QDOT_FN (function qualifiers) defined by the includer.
 */
#ifndef COLI_QDOT_H
#define COLI_QDOT_H

#include <stdint.h>

namespace coli {

/* Rearranges the 8 natural-order activation words of a block (codes 0..31,
 * little-endian) into the operand order of block_partial<BITS>. */
template <int BITS>
COLI_QDOT_FN void prep_activation(const uint32_t (&x)[8], uint32_t (&xa)[8])
{
    if constexpr (BITS == 8) {
        for (int i = 0; i < 8; ++i)
            xa[i] = x[i];
    } else if constexpr (BITS == 4) {
        /* weight word k holds elements 8k..8k+7: even elements in the high
         * nibbles, odd elements in the low nibbles. */
        for (int k = 0; k < 4; ++k) {
            xa[2 * k] = COLI_PERM(x[2 * k + 1], x[2 * k], 0x06040200u);     /* q0 q2 q4 q6 */
            xa[2 * k + 1] = COLI_PERM(x[2 * k + 1], x[2 * k], 0x07050301u); /* q1 q3 q5 q7 */
        }
    } else {
        /* weight word k holds elements 16k..16k+15; field r of byte j is
         * element 16k + 4j + r. Operand r collects byte r of the four
         * activation words of the group (a 4x4 byte transpose). */
        for (int k = 0; k < 2; ++k) {
            uint32_t a = x[4 * k], b = x[4 * k + 1], c = x[4 * k + 2], d = x[4 * k + 3];
            uint32_t ab_lo = COLI_PERM(b, a, 0x05010400u); /* a0 b0 a1 b1 */
            uint32_t ab_hi = COLI_PERM(b, a, 0x07030602u); /* a2 b2 a3 b3 */
            uint32_t cd_lo = COLI_PERM(d, c, 0x05010400u); /* c0 d0 c1 d1 */
            uint32_t cd_hi = COLI_PERM(d, c, 0x07030602u); /* c2 d2 c3 d3 */
            xa[4 * k + 0] = COLI_PERM(cd_lo, ab_lo, 0x05040100u); /* a0 b0 c0 d0 */
            xa[4 * k + 1] = COLI_PERM(cd_lo, ab_lo, 0x07060302u); /* a1 b1 c1 d1 */
            xa[4 * k + 2] = COLI_PERM(cd_hi, ab_hi, 0x05040100u); /* a2 b2 c2 d2 */
            xa[4 * k + 3] = COLI_PERM(cd_hi, ab_hi, 0x07060302u); /* a3 b3 c3 d3 */
        }
    }
}

/* Exact block partial: sum over the block's 32 elements of weight code times
 * activation code.  w: the block's BITS packed words; xa: prep_activation. */
template <int BITS>
COLI_QDOT_FN int32_t block_partial(const uint32_t* w, const uint32_t (&xa)[8])
{
    int32_t s = 0;
    if constexpr (BITS == 8) {
        for (int i = 0; i < 8; ++i)
            s = COLI_SDOT4(w[i], xa[i], s);
        return s;
    } else if constexpr (BITS == 4) {
        for (int k = 0; k < 4; ++k) {
            uint32_t hi = w[k] & 0xF0F0F0F0u;        /* 16 * even elements */
            uint32_t lo = (w[k] << 4) & 0xF0F0F0F0u; /* 16 * odd elements  */
            s = COLI_SDOT4(hi, xa[2 * k], s);
            s = COLI_SDOT4(lo, xa[2 * k + 1], s);
        }
        return s >> 4;
    } else {
        for (int k = 0; k < 2; ++k)
            for (int r = 0; r < 4; ++r)
                s = COLI_SDOT4((w[k] << (2 * r)) & 0xC0C0C0C0u, xa[4 * k + r], s);
        return s >> 6;
    }
}

/* Activation operands of block_dot<BITS>: int8 and int2 as prep_activation;
 * int4 as the two nibble planes, word 2k the h plane and word 2k+1 the l
 * plane of weight word k (nibble 2j+1 of a weight word is element 2j, nibble
 * 2j element 2j+1 of its eight). */
template <int BITS>
COLI_QDOT_FN void prep_dot(const uint32_t (&x)[8], uint32_t (&xa)[8])
{
    if constexpr (BITS != 4) {
        prep_activation<BITS>(x, xa);
    } else {
        for (int k = 0; k < 4; ++k) {
            const uint32_t ev = COLI_PERM(x[2 * k + 1], x[2 * k], 0x06040200u); /* e0 e2 e4 e6 */
            const uint32_t od = COLI_PERM(x[2 * k + 1], x[2 * k], 0x07050301u); /* e1 e3 e5 e7 */
            /* h: the high nibble of each code; l: its low nibble minus 8 */
            xa[2 * k] = (ev & 0xF0F0F0F0u) | ((od >> 4) & 0x0F0F0F0Fu);
            xa[2 * k + 1] = (((ev << 4) & 0xF0F0F0F0u) | (od & 0x0F0F0F0Fu)) ^ 0x88888888u;
        }
    }
}

/* Exact block partial of the VALU kernels (the same value as block_partial);
 * xa: prep_dot. */
template <int BITS>
COLI_QDOT_FN int32_t block_dot(const uint32_t* w, const uint32_t (&xa)[8])
{
    if constexpr (BITS != 4) {
        return block_partial<BITS>(w, xa);
    } else {
        int32_t sh = 0, sl = 0, sq = 0;
        for (int k = 0; k < 4; ++k) {
            sh = COLI_SDOT8(w[k], xa[2 * k], sh);
            sl = COLI_SDOT8(w[k], xa[2 * k + 1], sl);
            sq = COLI_SDOT8(w[k], 0x11111111u, sq); /* sum of the word's codes */
        }
        return ((2 * sh + sq) << 3) + sl;
    }
}

} // namespace coli

#endif
