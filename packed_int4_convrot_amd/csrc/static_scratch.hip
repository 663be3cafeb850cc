// Device scratch owned by the library, for the entry point that allocates
// nothing (ck_w4a4_linear_noalloc): the rotate-quant codes and row scales of
// the whole linear live in a fixed device array instead of a caller workspace.
//
// The array is a file-scope __device__ variable, so the HIP runtime places one
// copy on every GPU that loads this code object and keeps it until the
// process ends.  In host code its name is only a host-side handle: the device
// address of the copy on the current GPU comes from hipGetSymbolAddress, looked
// up once per device on the first call made with that device current, and that
// address (never the name) is what kernels and copies are given.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static constexpr size_t kScratchBytes = ck::kStaticScratchBytes;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace ck {
namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void *g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

int static_scratch(void *stream, void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return (int)e;
    if (dev < 0 || dev >= kMaxDevices)
        return (int)hipErrorInvalidDevice;
    if (stream) {
        // The address is the current device's copy: a stream of another device
        // would run its kernels against memory of the wrong GPU.
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev);
        if (e != hipSuccess)
            return (int)e;
        if (sdev != dev)
            return (int)hipErrorInvalidDevice;
    }
    std::call_once(g_once[dev], [dev] {
        g_err[dev] = hipGetSymbolAddress(&g_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_err[dev] != hipSuccess)
        return (int)g_err[dev];
    *ptr = g_ptr[dev];
    return 0;
}

}  // namespace ck
