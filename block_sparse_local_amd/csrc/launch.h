// launch.h -- what the C-ABI layer hands to the kernel launchers (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {

// One forward call, after argument validation.  Padded layout: cu_seqlens is
// nullptr and n is the buffer length.  Packed layout: cu_seqlens is set, n is
// the longest sequence the grid must cover and tokens the rows in the buffer.
struct Launch {
    const void *q, *k, *v;
    void *o;
    const int32_t *seqlens;    // device; nullptr = every sequence is n long
    const int32_t *cu_seqlens; // device, batch + 1 offsets (packed layout only)
    float *lse;                // device or nullptr
    int32_t *active;           // trace outputs (nullptr unless traced)
    uint32_t *masks;
    int32_t batch, heads, n, head_dim, radius;
    int32_t tokens;
    int32_t window; // 0: block band; >= 1: token window (radius = ceil(window / 32))
    bool causal;
    float scale; // already resolved (> 0)
    hipStream_t stream;
};

// Each returns hipSuccess or the error hipGetLastError reported for its launch.
hipError_t launch_fwd_bf16(const Launch &a);
hipError_t launch_fwd_f32(const Launch &a);

} // namespace bsl
