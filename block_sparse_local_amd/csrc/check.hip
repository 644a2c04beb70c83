// check.hip -- debug validators for the per-sequence lengths and packed
// offsets the forward reads from device memory, gfx950.
//
// The forward clamps every length into [0, n] and every offset into
// [0, tokens] on the device, so a bad value can never send an access out of
// bounds; it silently changes which rows are attended instead.  These checks
// report such values without a host round trip: one workgroup scans the array
// and writes {number of bad entries, index of the first one or -1} to a
// two-int32 device result.  Lengths follow the NucleoByte project page,
// section 2, item 2 ("Dynamic Ceiling Hardware Alignment"): each sequence
// fits its batch's padded length n.
#include "check.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {
namespace {

constexpr int TPB = 256;

// mode 0: lengths, bad when outside [0, limit].  mode 1: offsets (count + 1 of
// them), bad at index 0 when nonzero, at index b > 0 when below entry b - 1 or
// above limit.
__global__ void __launch_bounds__(TPB) check_kernel(const int32_t *v, int32_t count, int32_t limit,
                                                    int mode, int32_t *out)
{
    __shared__ int32_t bad, first;
    if (threadIdx.x == 0) {
        bad = 0;
        first = 0x7fffffff;
    }
    __syncthreads();
    const int32_t entries = mode == 0 ? count : count + 1;
    for (int32_t b = threadIdx.x; b < entries; b += TPB) {
        const int32_t x = v[b];
        bool wrong;
        if (mode == 0)
            wrong = x < 0 || x > limit;
        else
            wrong = b == 0 ? x != 0 : (x < v[b - 1] || x > limit);
        if (wrong) {
            atomicAdd(&bad, 1);
            atomicMin(&first, b);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        out[0] = bad;
        out[1] = bad ? first : -1;
    }
}

} // namespace

hipError_t launch_check(const int32_t *v, int32_t count, int32_t limit, int mode, int32_t *out,
                        hipStream_t stream)
{
    hipLaunchKernelGGL(check_kernel, dim3(1), dim3(TPB), 0, stream, v, count, limit, mode, out);
    return hipGetLastError();
}

} // namespace bsl
