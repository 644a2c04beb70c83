// fake_device.h -- a host-only stand-in for the HIP runtime calls and kernel
// launchers that bsl_api.cpp links against, so the C-ABI layer can be built
// with the host sanitizers and driven on a machine without a GPU.
//
// TEST INFRASTRUCTURE: linked only into tests/host/abi_host_test.cpp.  The
// launchers never touch the buffers they are given; they count calls and keep
// a copy of the last launch description for the test to inspect.
#pragma once

#include "bwd_launch.h"
#include "check.h"
#include "kmer_launch.h"
#include "launch.h"
#include "scratch.h"

namespace fake {

struct State {
    int current_device = 0;            // what hipGetDevice reports
    const char *arch = "gfx950:sramecc+:xnack-"; // gcnArchName of every device
    hipError_t launch_result = hipSuccess;       // what every launcher returns
    int fwd_bf16 = 0, fwd_f32 = 0, bwd_bf16 = 0, bwd_valu = 0, kmer = 0, check = 0;
    int scratch_lookups = 0;           // scratch_setup calls that did a lookup
    float *scratch = nullptr;          // the workspace "address" of every device
    bool last_bwd_valu_bf16 = false;
    bsl::Launch last_fwd{};
    bsl::BwdLaunch last_bwd{};
    bsl::KmerLaunch last_kmer{};
    int launches() const { return fwd_bf16 + fwd_f32 + bwd_bf16 + bwd_valu + kmer + check; }
};

State &state();

} // namespace fake
