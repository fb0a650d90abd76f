// kvq_scratch.hip -- the library's own device scratch for callers that
// cannot allocate (kvq_append_attend_static): a file-scope device array of
// fixed size that holds the decode attention's split partials instead of the
// workspace's partials region.
//
// Host code never passes the array's name to a kernel (on the host it is
// only a stand-in symbol): the device address is looked up once per device
// with hipGetSymbolAddress, with that device current, and kept in a table.
// Each device holds its own copy of the array until the process ends; every
// call on a device shares it, so calls that overlap on one device race.
#include "kvq_internal.h"

#include <mutex>

namespace kvqi {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int device, void** out)
{
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_ptr[device]) {
        int cur = -1;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess)
            return e;
        if (cur != device)
            return hipErrorInvalidDevice;  // the caller makes `device` current
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_ptr[device] = ptr;
    }
    *out = g_ptr[device];
    return hipSuccess;
}

}  // namespace kvqi
