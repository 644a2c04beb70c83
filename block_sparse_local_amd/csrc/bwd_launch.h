// bwd_launch.h -- what the C-ABI layer hands to the backward launcher (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {

// One backward call, after argument validation.
struct BwdLaunch {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    const int32_t *seqlens;    // padded layout; nullptr = every sequence is n long
    const int32_t *cu_seqlens; // packed layout: batch + 1 offsets (else nullptr)
    void *dq, *dk, *dv;
    float *delta; // caller's workspace, [batch][heads][n] (packed: [heads][tokens])
    int32_t batch, heads, n, head_dim, radius;
    int32_t tokens; // packed layout: rows in the buffers (n: the longest sequence)
    int32_t window; // 0: block band; >= 1: token window (radius = ceil(window / 32))
    bool causal;
    float scale;
    hipStream_t stream;
};

hipError_t launch_bwd_bf16(const BwdLaunch &a);
// The vector-ALU backward: fp32 plans, and bf16 plans at head_dim 32 (bf16 = true).
hipError_t launch_bwd_valu(const BwdLaunch &a, bool bf16);

} // namespace bsl
