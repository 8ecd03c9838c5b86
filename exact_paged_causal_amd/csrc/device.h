// device.h -- small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atlas {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// DPP controls (GFX9 data-parallel primitives; operate inside 16-lane rows).
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int Ctrl>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of Lanes (4, 8 or 16) lanes; every lane gets the total.
template <int Lanes>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp<kDppQuadSwap1>(x);
    x += dpp<kDppQuadSwap2>(x);
    if constexpr (Lanes >= 8)
        x += dpp<kDppRowHalfMirror>(x);
    if constexpr (Lanes >= 16)
        x += dpp<kDppRowMirror>(x);
    return x;
}

template <int Lanes>
__device__ __forceinline__ float group_max(float x)
{
    x = fmaxf(x, dpp<kDppQuadSwap1>(x));
    x = fmaxf(x, dpp<kDppQuadSwap2>(x));
    if constexpr (Lanes >= 8)
        x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
    if constexpr (Lanes >= 16)
        x = fmaxf(x, dpp<kDppRowMirror>(x));
    return x;
}

// Hardware 2^x (v_exp_f32): exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Ordinary 16-byte load through a native vector type (a uint4 dereference
// can keep a kernel's register buffers from being promoted to registers).
__device__ __forceinline__ uint4 load16(const void *p)
{
    typedef uint32_t u32x4_ld __attribute__((ext_vector_type(4)));
    const u32x4_ld v = *reinterpret_cast<const u32x4_ld *>(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load marked non-temporal: K/V rows a decode pass reads once stream
// past the caches instead of displacing lines other work reuses (measured on
// the long-context decode: the fold runs about 4 % faster).
__device__ __forceinline__ uint4 stream_load16(const void *p)
{
    typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
    const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// c * tanh(x * k) from one hardware exponential and one reciprocal, through
// tanh(y) = 1 - 2 / (e^(2y) + 1) with the constants folded:
// c - 2c / (2^(x * 2k log2 e) + 1).  Saturates to +-c (2^+big = inf, rcp(inf)
// = 0).  Absolute error of the tanh factor below 1e-6 (two hardware ops of
// about one ulp each on a value in (0, 1), plus two roundings).
__device__ __forceinline__ float scaled_tanh_fast(float x, float k2log2e, float c, float neg2c)
{
    const float e = __builtin_amdgcn_exp2f(x * k2log2e);
    return fmaf(neg2c, __builtin_amdgcn_rcpf(e + 1.0f), c);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

}  // namespace atlas
