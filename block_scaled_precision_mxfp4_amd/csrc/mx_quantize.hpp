// One 32-element block of a bf16 row -> MXFP4 (E2M1 codes + E8M0 scale),
// shared by the activation quantizer and the GEMV that quantizes its single
// A row on load.  The rule (OCP Microscaling Formats v1.0, section 6.3):
// scale exponent X = floor(log2 max|v|) - 2 clamped to [-127, 127]; each
// element v / 2^X rounded to the nearest E2M1 value, ties to the even
// mantissa, saturating at 6, sign kept; a block holding a NaN or an infinity
// gets scale 0xFF and codes 0.
#pragma once

#include "mx_device.hpp"

namespace mx {

// Encode one 32-block: x holds this lane's 8 bf16 (a quarter of the block);
// the four lanes of the block combine their maximum and NaN/inf flag.
__device__ __forceinline__ void quantize_quarter(v4i x, uint32_t &word, uint8_t &scale)
{
    // bf16 magnitude bits order like the values for finite inputs; an
    // all-ones exponent field is an infinity or a NaN
    uint32_t amag = 0, special = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t hb = ((uint32_t)x[w] >> (16 * h)) & 0xFFFFu;
            special |= (hb & 0x7F80u) == 0x7F80u;
            amag = max(amag, hb & 0x7FFFu);
        }
    }
    // the block's four lanes are one aligned quad: quad permutes (lane ^ 1,
    // lane ^ 2) exchange within it without going through LDS
    amag = max(amag, (uint32_t)__builtin_amdgcn_mov_dpp((int)amag, 0xB1, 0xF, 0xF, true));
    amag = max(amag, (uint32_t)__builtin_amdgcn_mov_dpp((int)amag, 0x4E, 0xF, 0xF, true));
    special |= (uint32_t)__builtin_amdgcn_mov_dpp((int)special, 0xB1, 0xF, 0xF, true);
    special |= (uint32_t)__builtin_amdgcn_mov_dpp((int)special, 0x4E, 0xF, 0xF, true);

    // floor(log2 amax) from the bf16 fields (subnormal: from the top set
    // mantissa bit), then the scale exponent
    int xs = -127;
    if (amag != 0) {
        const int ef = (int)(amag >> 7);
        const int fl = ef > 0 ? ef - 127 : -133 + (31 - __builtin_clz(amag & 0x7Fu));
        xs = min(127, max(-127, fl - 2));
    }
    word = 0;
    if (!special && xs > -127) {
        // v_cvt_scalef32_pk_fp4_bf16: two bf16 divided by the scale, rounded
        // to nearest even E2M1 with saturation at 6, sign kept -- the rule
        // above, measured equal on every finite input tried; one instruction
        // per pair, byte w of the word holds elements 2w (low nibble), 2w+1
        // (the pairs are formed from the whole 16 bytes viewed as eight
        // bf16: a bit cast of single extracted words was folded onto word 0)
        typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
        typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
        const v8bf_t e = __builtin_bit_cast(v8bf_t, x);
        const float sc = __uint_as_float((uint32_t)(xs + 127) << 23);  // 2^xs, a normal float
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v2bf_t{e[0], e[1]}, sc, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v2bf_t{e[2], e[3]}, sc, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v2bf_t{e[4], e[5]}, sc, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(word, v2bf_t{e[6], e[7]}, sc, 3);
    } else if (!special) {
        // scale 2^-127 is not a normal float: encode in software
#pragma unroll
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t hb = ((uint32_t)x[w] >> (16 * h)) & 0xFFFFu;
                const float s = ldexpf(__uint_as_float(hb << 16), -xs);  // exact scaling
                const float m = fabsf(s);
                uint32_t c;
                if (m >= 6.0f)
                    c = 7u;  // saturate (no E2M1 value above 6)
                else if (m < 2.0f)
                    c = (uint32_t)rintf(m * 2.0f);  // steps of 1/2: codes 0..4
                else if (m < 4.0f)
                    c = (uint32_t)rintf(m) + 2u;  // 2, 3, 4 -> codes 4, 5, 6
                else
                    c = (uint32_t)rintf(m * 0.5f) + 4u;  // 4, 6 -> codes 6, 7
                c |= (hb >> 12) & 8u;  // sign bit of the input
                word |= c << (4 * (2 * w + h));
            }
        }
    }
    scale = special ? (uint8_t)0xFF : (uint8_t)(xs + 127);
}

}  // namespace mx
