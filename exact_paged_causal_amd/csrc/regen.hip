// regen.hip -- on-device deterministic page regenerator.
//
// Writes whole (page, K/V head) slabs of regenerated K and V (row-major
// K[token][dim], V[token][dim]) into the arenas; the generator itself is in
// philox.h.  One thread produces four consecutive dims of one token for both
// K and V, so stores are 16-byte (fp32) or 8-byte (bf16) and contiguous
// across a wave.  The work is ALU-bound (20 32x32->64-bit multiplies plus
// log/sqrt/sincospi per four values).
#include "device.h"
#include "kernels.h"
#include "philox.h"

namespace atlas {
namespace {

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
    const int64_t elem = ((((int64_t)phys * a.hkv + h) << a.page_shift) + t) * D + quad * 4;

#pragma unroll
    for (int tensor = 1; tensor <= 2; ++tensor) {
        float z[4];
        regen_quad(a.seed, (uint32_t)a.layer, (uint32_t)seq, (uint32_t)tensor, (uint32_t)h, token, (uint32_t)quad, z);
        const float z0 = z[0], z1 = z[1], z2 = z[2], z3 = z[3];
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
            const f32x4 zv = {z0, z1, z2, z3};
            __builtin_nontemporal_store(zv, reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(arena) + elem));
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
