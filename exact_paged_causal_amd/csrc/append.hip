// append.hip -- write new tokens' K/V rows into their pages.
//
// The decode step's cache update (CPUAttn README: cache-backed decode streams
// grow by one token per step): token t of sequence b, at position
// p = start_pos[b] + t, goes to row p % P of physical page
// page_table[b][p / P] for every K/V head.  One thread moves one 16-byte
// piece of one (token, head) row of K and the same piece of V: reads are
// contiguous across a wave, and so are the writes within a row.  Rows whose
// page id or position is out of range are skipped.
#include "device.h"
#include "kernels.h"

namespace atlas {
namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a, int64_t total)
{
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= total)
        return;
    const int pieces = a.row_bytes / 16;                 // 16-byte pieces per row
    const int64_t row = gid / pieces;                    // (b, t, h) row of the new tokens
    const int piece = (int)(gid - row * pieces);
    const int h = (int)(row % a.hkv);
    const int64_t bt = row / a.hkv;
    const int t = (int)(bt % a.n_new);
    const int b = (int)(bt / a.n_new);
    const int64_t pos = (int64_t)a.start_pos[b] + t;
    if (pos < 0 || pos >= ((int64_t)a.max_pages << a.page_shift))
        return;
    const int32_t pid = a.page_table[(int64_t)b * a.max_pages + (pos >> a.page_shift)];
    if ((unsigned)pid >= (unsigned)a.num_phys)
        return;
    const int64_t dst = ((((int64_t)pid * a.hkv + h) << a.page_shift) + (pos & ((1 << a.page_shift) - 1))) *
                            a.row_bytes + piece * 16;
    const int64_t src = row * a.row_bytes + piece * 16;
    const uint4 kv = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.k_new) + src);
    const uint4 vv = *reinterpret_cast<const uint4 *>(static_cast<const char *>(a.v_new) + src);
    *reinterpret_cast<uint4 *>(static_cast<char *>(a.k_pages) + dst) = kv;
    *reinterpret_cast<uint4 *>(static_cast<char *>(a.v_pages) + dst) = vv;
}

}  // namespace

hipError_t launch_append(const AppendArgs &a, hipStream_t stream)
{
    const int64_t total = (int64_t)a.batch * a.n_new * a.hkv * (a.row_bytes / 16);
    if (total <= 0)
        return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, total);
    return hipGetLastError();
}

}  // namespace atlas
