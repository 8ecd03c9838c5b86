// philox.h -- the page regenerator's value generator, shared by the
// regenerator kernel (regen.hip) and the fold that regenerates cold pages in
// registers (split_valu.hip), so both produce the same bits.
//
// CFR-Atlas README ("Minimal integration", "Core contract"): a cold page is
// replayed as row-major K[token][dim] / V[token][dim] rows of one (layer, K/V
// head, token range), and attention over replayed pages must equal attention
// over stored ones.  The pages do not show the reference adapter's
// generator; this one is a counter-based hash, so any value can be rebuilt
// independently and in any order:
//   counter = (token, dim / 4, head | tensor << 30, layer | seq << 16),
//   key = seed, words = Philox4x32-10(counter, key)  (Salmon, Moraes, Dror,
//   Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11),
// then the Box-Muller transform (Box and Muller, 1958) of word pairs:
//   u(x) = (floor(x / 512) + 1/2) 2^-23       (exact in fp32, inside (0,1))
//   dims 4k, 4k+1   = r cos(2 pi u(w1)), r sin(2 pi u(w1)),  r = sqrt(-2 ln u(w0))
//   dims 4k+2, 4k+3 = the same with words w2, w3.
// tensor 1 is K, 2 is V.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atlas {

struct PhiloxWords {
    uint32_t w0, w1, w2, w3;
};

// Philox4x32-10: ten rounds of the Philox S-box.  Round: multiply word 0 by
// 0xD2511F53 and word 2 by 0xCD9E8D57 (64-bit products); new words are
// (hi2 ^ w1 ^ k0, lo2, hi0 ^ w3 ^ k1, lo0); between rounds the key advances by
// the Weyl increments 0x9E3779B9 and 0xBB67AE85.
__device__ __forceinline__ PhiloxWords philox10(PhiloxWords c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.w0;
        const uint64_t p2 = (uint64_t)0xCD9E8D57u * c.w2;
        // Three-input XORs as one gfx950 bitop3 each (truth table 0x96).
        const uint32_t x0 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p2 >> 32), c.w1, k0, 0x96);
        const uint32_t x2 = (uint32_t)__builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w3, k1, 0x96);
        const PhiloxWords n{x0, (uint32_t)p2, x2, (uint32_t)p0};
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ __forceinline__ float philox_unit_open(uint32_t x)
{
    // (floor(x / 512) + 1/2) * 2^-23 = (2 floor(x/512) + 1) * 2^-24: 24 bits, exact.
    // The top 23 bits of x become the mantissa of a float in [1, 2) (one
    // funnel shift: 0x7F above x, shifted right by 9), and subtracting
    // 1 - 2^-24 leaves exactly (x>>9) 2^-23 + 2^-24 (the difference is
    // representable, so the subtraction is exact).
    return __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, x, 9u)) - 0x1.fffffep-1f;
}

__device__ __forceinline__ void box_muller(uint32_t wr, uint32_t wa, float &zc, float &zs)
{
    // -2 ln u = -2 ln 2 * log2 u, with log2 and the square root on the
    // hardware units.
    const float r = __builtin_amdgcn_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(philox_unit_open(wr)));
    // sin / cos of 2 pi u on the hardware units, whose argument is in
    // revolutions (u itself, no range reduction needed in (0, 1)).
    const float ua = philox_unit_open(wa);
    const float sn = __builtin_amdgcn_sinf(ua);
    const float cs = __builtin_amdgcn_cosf(ua);
    zc = r * cs;
    zs = r * sn;
}

// The four values of dims 4*quad .. 4*quad+3 of one row.
// tensor: 1 = K, 2 = V.
__device__ __forceinline__ void regen_quad(uint64_t seed, uint32_t layer, uint32_t seq, uint32_t tensor,
                                           uint32_t head, uint32_t token, uint32_t quad, float z[4])
{
    const PhiloxWords w = philox10(PhiloxWords{token, quad, head | (tensor << 30), layer | (seq << 16)},
                                   (uint32_t)seed, (uint32_t)(seed >> 32));
    box_muller(w.w0, w.w1, z[0], z[1]);
    box_muller(w.w2, w.w3, z[2], z[3]);
}

}  // namespace atlas
