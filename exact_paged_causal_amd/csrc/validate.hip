// validate.hip -- validation-mode scan for NaN/Inf in the inputs a call reads.
//
// The CFR-Atlas README ("Validation and hardening") rejects non-finite
// inputs before they reach the cache.  In validation mode the C ABI runs this
// scan first: every query element, and every K/V element of the rows each
// sequence's context covers (rows past the context are never read and are
// not scanned).  For the tiled prefills it also flags V values outside the
// fp16 range of their P.V products (the fp32 kernel scales Q and K rows into
// that range itself).  Hits set bits of a flag word, which the host reads
// back.
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

template <typename E>
__device__ __forceinline__ bool finite_elem(E x);

template <typename E>
__device__ __forceinline__ bool beyond_f16(E x);

template <>
__device__ __forceinline__ bool beyond_f16<float>(float x)
{
    return fabsf(x) > 65504.0f;
}

template <>
__device__ __forceinline__ bool beyond_f16<uint16_t>(uint16_t x)
{
    return fabsf(__uint_as_float((uint32_t)x << 16)) > 65504.0f;
}

template <>
__device__ __forceinline__ bool finite_elem<float>(float x)
{
    return (__float_as_uint(x) & 0x7F800000u) != 0x7F800000u;
}

template <>
__device__ __forceinline__ bool finite_elem<uint16_t>(uint16_t x)
{
    return (x & 0x7F80u) != 0x7F80u;
}

template <typename EQ, typename E>
__global__ __launch_bounds__(256) void scan_kernel(ScanArgs a)
{
    // blockIdx.x: logical page index (last one: the queries), blockIdx.y: sequence
    const int b = blockIdx.y;
    const int lp = blockIdx.x;
    int ctx = a.context_lens[b];
    ctx = ctx < 0 ? 0 : (ctx > a.max_context ? a.max_context : ctx);
    bool bad = false;
    bool wide = false;
    if (lp == a.max_pages) {
        const int64_t n = (int64_t)a.q_len * a.hq * a.head_dim;
        const EQ *q = reinterpret_cast<const EQ *>(a.q) + (int64_t)b * n;
        for (int64_t i = threadIdx.x; i < n; i += 256) {
            bad |= !finite_elem<EQ>(q[i]);
        }
    } else {
        const int P = 1 << a.page_shift;
        const int rows = ctx - lp * P < P ? ctx - lp * P : P;
        if (rows > 0) {
            int pid = a.page_table[(int64_t)b * a.max_pages + lp];
            if ((unsigned)pid < (unsigned)a.num_phys) {
                const int64_t per_head = (int64_t)P * a.head_dim;
                const int64_t n = (int64_t)a.hkv * rows * a.head_dim;
                for (int64_t i = threadIdx.x; i < n; i += 256) {
                    const int64_t h = i / ((int64_t)rows * a.head_dim);
                    const int64_t rest = i - h * rows * a.head_dim;
                    const int64_t off = ((int64_t)pid * a.hkv + h) * per_head + rest;
                    const E kk = reinterpret_cast<const E *>(a.k_pages)[off];
                    const E vv = reinterpret_cast<const E *>(a.v_pages)[off];
                    bad |= !finite_elem<E>(kk);
                    bad |= !finite_elem<E>(vv);
                    wide |= a.check_f16 != 0 && beyond_f16<E>(vv);
                }
            }
        }
    }
    if (bad)
        atomicOr(a.flag, 1);
    if (wide)
        atomicOr(a.flag, 2);
}

}  // namespace

hipError_t launch_scan(const ScanArgs &a, int q_dtype, int kv_dtype, hipStream_t stream)
{
    dim3 grid(a.max_pages + 1, a.batch);
    if (kv_dtype == 0)
        hipLaunchKernelGGL((scan_kernel<float, float>), grid, dim3(256), 0, stream, a);
    else if (q_dtype == 0)
        hipLaunchKernelGGL((scan_kernel<float, uint16_t>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((scan_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace atlas
