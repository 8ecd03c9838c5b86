// regen.hip -- on-device deterministic page regenerator.
//
// Writes whole (page, K/V head) slabs of regenerated K and V (row-major
// K[token][dim], V[token][dim]) into the arenas; the generator itself is in
// philox.h.  One thread produces four consecutive dims of one token for both
// K and V, so stores are 16-byte (fp32) or 8-byte (bf16) and contiguous
// across a wave.  The work is ALU-bound (20 32x32->64-bit multiplies plus
// log2/sqrt/sin/cos per four values); the grid's x dimension covers the items
// of one job and y the jobs, so no thread divides by the job size (a 64-bit
// division per thread cost about 7 % of the kernel).
#include "device.h"
#include "kernels.h"
#include "philox.h"

namespace atlas {
namespace {

template <int D, bool BF16>
__global__ __launch_bounds__(256) void regen_kernel(RegenArgs a, int items_per_job)
{
    constexpr int Q = D / 4;  // 4-dim groups per row
    // x: the items of one job (no division by the job size); y: jobs, with a
    // stride of the grid's height when there are more jobs than it holds.
    const int item = (int)blockIdx.x * 256 + (int)threadIdx.x;
    if (item >= items_per_job)
        return;
    const int quad = item % Q;
    const int th = item / Q;                      // head * P + token-in-page
    const int t = th & ((1 << a.page_shift) - 1);
    const int h = th >> a.page_shift;
    for (int64_t job = blockIdx.y; job < a.n_jobs; job += gridDim.y) {
        const int32_t seq = a.jobs[job * 3 + 0];
        const int32_t lp = a.jobs[job * 3 + 1];
        const int32_t phys = a.jobs[job * 3 + 2];
        // The generator's counter holds 16 bits of the sequence key: keys
        // outside [0, 65536) would alias another sequence's values.
        if ((unsigned)seq >= 65536u || lp < 0 || (unsigned)phys >= (unsigned)a.num_phys)
            continue;
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
}

}  // namespace

hipError_t launch_regen(const RegenArgs &a, int dtype, hipStream_t stream)
{
    if (a.n_jobs <= 0)
        return hipSuccess;
    const int64_t items_per_job = ((int64_t)a.hkv << a.page_shift) * (a.head_dim / 4);
    if (items_per_job > 0x7FFFFF00)
        return hipErrorInvalidValue;
    const int64_t jobs_y = a.n_jobs < 65535 ? a.n_jobs : 65535;
    dim3 grid((unsigned)((items_per_job + 255) / 256), (unsigned)jobs_y);
    const int ipj = (int)items_per_job;
    if (a.head_dim == 64) {
        if (dtype == 0)
            hipLaunchKernelGGL((regen_kernel<64, false>), grid, dim3(256), 0, stream, a, ipj);
        else
            hipLaunchKernelGGL((regen_kernel<64, true>), grid, dim3(256), 0, stream, a, ipj);
    } else {
        if (dtype == 0)
            hipLaunchKernelGGL((regen_kernel<128, false>), grid, dim3(256), 0, stream, a, ipj);
        else
            hipLaunchKernelGGL((regen_kernel<128, true>), grid, dim3(256), 0, stream, a, ipj);
    }
    return hipGetLastError();
}

}  // namespace atlas
