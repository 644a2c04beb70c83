// scratch.hip -- the fixed device workspace behind bsl_backward_noalloc.
//
// The backward pass keeps one float per row (D_t = dO_t . O_t) between its two
// kernels.  bsl_backward takes that buffer from the caller; callers that
// cannot allocate (code under graph capture, tight serving loops, harnesses
// that forbid hipMalloc) use bsl_backward_noalloc, which keeps it here, in a
// file-scope device array the runtime places on every device when it loads
// the code object.  Each device has its own copy at its own address; host code
// must use the address hipGetSymbolAddress returns on that device (the array's
// name on the host is only a handle for the lookup), so the address is looked
// up once per device, with that device current, and kept.
#include "scratch.h"

#include <mutex>

namespace bsl {

static __device__ __align__(256) float scratch[SCRATCH_FLOATS];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mutex;
float *g_address[MAX_DEVICES] = {};
} // namespace

hipError_t scratch_setup(int device)
{
    if (device < 0 || device >= MAX_DEVICES)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (g_address[device])
        return hipSuccess;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess)
        return e;
    g_address[device] = (float *)p;
    return hipSuccess;
}

float *scratch_on(int device)
{
    if (device < 0 || device >= MAX_DEVICES)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_mutex);
    return g_address[device];
}

} // namespace bsl
