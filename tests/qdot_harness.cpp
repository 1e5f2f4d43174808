// CPU harness for the GPU library's container unpacking (csrc/qdot.h): the
// same template code, compiled with g++ against emulations of the three gfx950
// instructions it uses, so the layout logic can be checked without a GPU.
#include <stdint.h>
#include <string.h>

// v_perm_b32: byte i of the result is byte sel[i] of the 8-byte value whose
// bytes 0..3 are s1 and bytes 4..7 are s0 (selectors 0..7 only are used).
static uint32_t emu_perm(uint32_t s0, uint32_t s1, uint32_t sel)
{
    uint64_t v = ((uint64_t)s0 << 32) | s1;
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
        uint32_t b = (sel >> (8 * i)) & 0xFF;
        r |= (uint32_t)((v >> (8 * b)) & 0xFF) << (8 * i);
    }
    return r;
}

// v_dot4_i32_i8: signed byte dot product plus accumulator.
static int32_t emu_sdot4(uint32_t a, uint32_t b, int32_t c)
{
    for (int i = 0; i < 4; ++i)
        c += (int32_t)(int8_t)(a >> (8 * i)) * (int32_t)(int8_t)(b >> (8 * i));
    return c;
}

// v_dot8_i32_i4: signed nibble dot product plus accumulator (nibble i of
// each operand is bits 4i+3..4i).
static int32_t emu_sdot8(uint32_t a, uint32_t b, int32_t c)
{
    for (int i = 0; i < 8; ++i) {
        const int32_t x = (int32_t)((a >> (4 * i)) & 15u), y = (int32_t)((b >> (4 * i)) & 15u);
        c += (x >= 8 ? x - 16 : x) * (y >= 8 ? y - 16 : y);
    }
    return c;
}

#define COLI_QDOT_FN static inline
#define COLI_PERM(a, b, s) emu_perm((a), (b), (s))
#define COLI_SDOT4(a, b, c) emu_sdot4((a), (b), (c))
#define COLI_SDOT8(a, b, c) emu_sdot8((a), (b), (c))
#include "../quantized_routed_expert_sigmoid_amd/csrc/qdot.h"

extern "C" int32_t harness_block_partial(int bits, const uint8_t* wblock, const int8_t* codes)
{
    uint32_t x[8], xa[8], w[8];
    memcpy(x, codes, 32);
    memcpy(w, wblock, 4 * bits);
    switch (bits) {
    case 8:
        coli::prep_activation<8>(x, xa);
        return coli::block_partial<8>(w, xa);
    case 4:
        coli::prep_activation<4>(x, xa);
        return coli::block_partial<4>(w, xa);
    default:
        coli::prep_activation<2>(x, xa);
        return coli::block_partial<2>(w, xa);
    }
}

// The VALU kernels' form (prep_dot / block_dot).
extern "C" int32_t harness_block_dot(int bits, const uint8_t* wblock, const int8_t* codes)
{
    uint32_t x[8], xa[8], w[8];
    memcpy(x, codes, 32);
    memcpy(w, wblock, 4 * bits);
    switch (bits) {
    case 8:
        coli::prep_dot<8>(x, xa);
        return coli::block_dot<8>(w, xa);
    case 4:
        coli::prep_dot<4>(x, xa);
        return coli::block_dot<4>(w, xa);
    default:
        coli::prep_dot<2>(x, xa);
        return coli::block_dot<2>(w, xa);
    }
}
