// regen.hip -- on-device deterministic page regenerator.
//
// CFR-Atlas README ("Minimal integration", "Core contract"): a cold page is
// replayed, as row-major K[token][dim] and V[token][dim] rows of one
// (layer, K/V head, token range), into scratch, and attention over replayed
// pages must equal attention over stored ones.  The pages do not show the
// reference adapter's generator; this one is a counter-based hash, so any
// page can be rebuilt independently and in any order:
//   counter = (token, dim / 4, head | tensor << 30, layer | seq << 16),
//   key = seed, words = Philox4x32-10(counter, key)  (Salmon, Moraes, Dror,
//   Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11),
// then the Box-Muller transform (Box and Muller, 1958) of word pairs:
//   u(x) = (floor(x / 512) + 1/2) 2^-23       (exact in fp32, inside (0,1))
//   dims 4k, 4k+1   = r cos(2 pi u(w1)), r sin(2 pi u(w1)),  r = sqrt(-2 ln u(w0))
//   dims 4k+2, 4k+3 = the same with words w2, w3.
// tensor 1 is K, 2 is V.  One thread produces four consecutive dims of one
// token for both K and V, so stores are 16-byte (fp32) or 8-byte (bf16) and
// contiguous across a wave.  The work is ALU-bound (20 32x32->64-bit
// multiplies plus log/sqrt/sincospi per four values).
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

struct Words {
    uint32_t w0, w1, w2, w3;
};

// Philox4x32-10: ten rounds of the Philox S-box.  Round: multiply word 0 by
// 0xD2511F53 and word 2 by 0xCD9E8D57 (64-bit products); new words are
// (hi2 ^ w1 ^ k0, lo2, hi0 ^ w3 ^ k1, lo0); between rounds the key advances by
// the Weyl increments 0x9E3779B9 and 0xBB67AE85.
__device__ __forceinline__ Words philox10(Words c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c.w0;
        const uint64_t p2 = (uint64_t)0xCD9E8D57u * c.w2;
        const Words n{(uint32_t)(p2 >> 32) ^ c.w1 ^ k0, (uint32_t)p2,
                      (uint32_t)(p0 >> 32) ^ c.w3 ^ k1, (uint32_t)p0};
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

__device__ __forceinline__ float unit_open(uint32_t x)
{
    // (floor(x / 512) + 1/2) * 2^-23 = (2 floor(x/512) + 1) * 2^-24: 24 bits, exact.
    return fmaf((float)(x >> 9), 0x1p-23f, 0x1p-24f);
}

__device__ __forceinline__ void box_muller(uint32_t wr, uint32_t wa, float &zc, float &zs)
{
    const float r = sqrtf(-2.0f * logf(unit_open(wr)));
    float sn, cs;
    sincospif(2.0f * unit_open(wa), &sn, &cs);
    zc = r * cs;
    zs = r * sn;
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void regen_kernel(RegenArgs a, int64_t items_per_job)
{
    constexpr int Q = D / 4;  // 4-dim groups per row
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t job = gid / items_per_job;
    if (job >= a.n_jobs)
        return;
    const int64_t item = gid - job * items_per_job;
    const int quad = (int)(item % Q);
    const int64_t th = item / Q;                  // head * P + token-in-page
    const int t = (int)(th & ((1 << a.page_shift) - 1));
    const int h = (int)(th >> a.page_shift);

    const int32_t seq = a.jobs[job * 3 + 0];
    const int32_t lp = a.jobs[job * 3 + 1];
    const int32_t phys = a.jobs[job * 3 + 2];
    if (seq < 0 || lp < 0 || (unsigned)phys >= (unsigned)a.num_phys)
        return;
    const uint32_t token = ((uint32_t)lp << a.page_shift) + (uint32_t)t;
    const uint32_t k0 = (uint32_t)a.seed, k1 = (uint32_t)(a.seed >> 32);
    const uint32_t w3 = (uint32_t)a.layer | ((uint32_t)seq << 16);
    const int64_t elem = ((((int64_t)phys * a.hkv + h) << a.page_shift) + t) * D + quad * 4;

#pragma unroll
    for (int tensor = 1; tensor <= 2; ++tensor) {
        const Words w = philox10(Words{token, (uint32_t)quad, (uint32_t)h | ((uint32_t)tensor << 30), w3},
                                 k0, k1);
        float z0, z1, z2, z3;
        box_muller(w.w0, w.w1, z0, z1);
        box_muller(w.w2, w.w3, z2, z3);
        // Non-temporal stores: the pages go straight to HBM while this
        // ALU-bound kernel runs, instead of sitting dirty in the last-level
        // cache and being written back while the attention pass reads.
        void *arena = tensor == 1 ? a.k_pages : a.v_pages;
        if constexpr (BF16) {
            typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
            const u32x2 packed = {f32_to_bf16_bits(z0) | (f32_to_bf16_bits(z1) << 16),
                                  f32_to_bf16_bits(z2) | (f32_to_bf16_bits(z3) << 16)};
            __builtin_nontemporal_store(packed, reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(arena) + elem));
        } else {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            const f32x4 z = {z0, z1, z2, z3};
            __builtin_nontemporal_store(z, reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(arena) + elem));
        }
    }
}

}  // namespace

hipError_t launch_regen(const RegenArgs &a, int dtype, hipStream_t stream)
{
    if (a.n_jobs <= 0)
        return hipSuccess;
    const int64_t items_per_job = ((int64_t)a.hkv << a.page_shift) * (a.head_dim / 4);
    const int64_t total = items_per_job * a.n_jobs;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    dim3 grid((unsigned)blocks);
    if (a.head_dim == 64) {
        if (dtype == 0)
            hipLaunchKernelGGL((regen_kernel<64, false>), grid, dim3(256), 0, stream, a, items_per_job);
        else
            hipLaunchKernelGGL((regen_kernel<64, true>), grid, dim3(256), 0, stream, a, items_per_job);
    } else {
        if (dtype == 0)
            hipLaunchKernelGGL((regen_kernel<128, false>), grid, dim3(256), 0, stream, a, items_per_job);
        else
            hipLaunchKernelGGL((regen_kernel<128, true>), grid, dim3(256), 0, stream, a, items_per_job);
    }
    return hipGetLastError();
}

}  // namespace atlas
