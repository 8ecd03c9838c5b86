// noalloc.hip -- atlas_attend_decode_noalloc: decode for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).
//
// atlas_attend_decode keeps its split partial states (running max, sum,
// unnormalised accumulator per output row and key span) in a workspace the
// caller allocates.  This entry point keeps them in `scratch`, a file-scope
// device array of kScratchBytes that each GPU the library runs on holds from
// the code object's load until the process ends; everything else is the same
// call (same kernels, same plan, same bits).  The array's host-side name is
// only a stand-in for the symbol: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and that
// address is what the kernels receive.  The partial states are fully written
// by the fold before the merge reads them, so nothing in the array has to
// start at zero.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/atlas.h"
#include "status.h"

namespace {

constexpr size_t kScratchBytes = ATLAS_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch[kMaxDevices];  // per device: the device address of `scratch` (null until looked up)

// Device address of this device's copy of `scratch`, looked up on the
// device's first call.
int32_t scratch_address(hipStream_t stream, void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return atlas::fail(ATLAS_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return atlas::fail(ATLAS_ERR_DEVICE, "device %d beyond the %d devices the scratch table covers", dev,
                           kMaxDevices);
    if (stream) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess)
            return atlas::fail(ATLAS_ERR_DEVICE, "hipStreamGetDevice: %s", hipGetErrorString(e));
        if (sdev != dev)
            return atlas::fail(ATLAS_ERR_DEVICE, "the stream belongs to device %d, the current device is %d",
                               (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return atlas::fail(ATLAS_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                               hipGetErrorString(e));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return ATLAS_OK;
}

bool validate_mode()
{
    const char *v = std::getenv("ATLAS_VALIDATE");
    return v && v[0] && std::strcmp(v, "0") != 0;
}

}  // namespace

extern "C" int32_t atlas_attend_decode_noalloc(const atlas_attn_args *args, void *stream)
{
    if (!args)
        return atlas::fail(ATLAS_ERR_NULL, "args is NULL");
    // Sizes first (host only): the partial states must fit the array.
    atlas_attn_args a = *args;
    a.workspace = nullptr;
    a.workspace_bytes = 0;
    const size_t need = atlas_decode_workspace_bytes(&a);
    if (need == SIZE_MAX)  // invalid arguments: the decode's own checks report them, launching nothing
        return atlas_attend_decode(&a, stream);
    if (need > kScratchBytes)
        return atlas::fail(ATLAS_ERR_WORKSPACE,
                           "this decode needs %zu bytes of partial states; the allocation-free entry point "
                           "holds at most %zu (use atlas_attend_decode with a workspace)",
                           need, kScratchBytes);
    if (validate_mode())
        return atlas::fail(ATLAS_ERR_UNSUPPORTED, "validation mode copies device arrays to host buffers; "
                                                  "use atlas_attend_decode");
    void *ptr = nullptr;
    const int32_t st = scratch_address(reinterpret_cast<hipStream_t>(stream), &ptr);
    if (st != ATLAS_OK)
        return st;
    a.workspace = ptr;
    a.workspace_bytes = kScratchBytes;
    return atlas_attend_decode(&a, stream);
}
