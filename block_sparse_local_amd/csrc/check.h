// check.h -- internal interface of the length / offset validator (check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {

// mode 0 checks count lengths against [0, limit]; mode 1 checks count + 1
// offsets (first 0, non-decreasing, at most limit).  Writes {bad entries,
// first bad index or -1} to out[2].
hipError_t launch_check(const int32_t *v, int32_t count, int32_t limit, int mode, int32_t *out,
                        hipStream_t stream);

} // namespace bsl
