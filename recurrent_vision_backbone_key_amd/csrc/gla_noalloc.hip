// gla_noalloc.hip -- the library-owned scratch array behind gla_fwd_noalloc.
//
// A caller that cannot allocate device memory (code under graph capture, a
// serving loop, a harness that forbids allocation) still needs the
// single-pass exchange area (counters, flags, segment aggregates) or the
// three-pass segment slots that gla_fwd keeps in the caller's workspace.  This
// file holds that area as one file-scope device array.  Every GPU the library
// runs on holds its own copy, at its own address, until the process ends; the
// host never uses the array's name as an address: the device address of each
// GPU's copy is looked up once, with that GPU current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gla.h"
#include "gla_launch.h"
#include "gla_plan.h"

namespace gla {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];     // device address of `scratch` on each device
bool g_ready[kMaxDevices];    // looked up and initialised (mark written)

}  // namespace

int scratch_for_device(int dev, void* stream, void** ptr)
{
    if (dev < 0 || dev >= kMaxDevices) return GLA_EHIP;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_ready[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return GLA_EHIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return GLA_EHIP;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return GLA_EHIP;
        }
        // counters, flags and error word start at zero (a device array is
        // zero-filled when the code object loads); the prefix is cleared and
        // the initialisation mark written on the first call's stream, ahead of
        // that call's kernels
        const int st = launch_workspace_init(p, GLA_PREFIX_BYTES, stream);
        if (st != GLA_OK) return st;
        g_ptr[dev] = p;
        g_ready[dev] = true;
    }
    *ptr = g_ptr[dev];
    return GLA_OK;
}

}  // namespace gla
