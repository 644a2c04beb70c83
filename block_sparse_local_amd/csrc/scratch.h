// scratch.h -- the library's one fixed device workspace (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace bsl {

// Floats in the workspace of bsl_backward_noalloc: 8 Mi floats = 32 MiB on each
// device, enough for the backward's row vector D of batch * heads * n up to
// 8,388,608 rows (the million-token shape: 8 heads x 2^20 rows).
constexpr size_t SCRATCH_FLOATS = size_t(8) << 20;

// Looks up, once per device, the device address of the workspace on the
// current device (call with that device current).  hipSuccess, or the error
// of the lookup.
hipError_t scratch_setup(int device);

// The address scratch_setup found for `device`, or nullptr if it has not run
// (or failed) there.
float *scratch_on(int device);

} // namespace bsl
