// fake_device.cpp -- definitions behind fake_device.h (host test only).
#include "fake_device.h"

#include <cstring>

namespace fake {
State &state()
{
    static State s;
    return s;
}
} // namespace fake

extern "C" {

hipError_t hipGetDevice(int *device)
{
    *device = fake::state().current_device;
    return hipSuccess;
}

hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_t *prop, int device)
{
    if (device < 0 || device > 7)
        return hipErrorInvalidDevice;
    std::memset(prop, 0, sizeof *prop);
    std::strncpy(prop->gcnArchName, fake::state().arch, sizeof prop->gcnArchName - 1);
    prop->multiProcessorCount = 256;
    return hipSuccess;
}

const char *hipGetErrorString(hipError_t e)
{
    return e == hipSuccess ? "hipSuccess" : "fake launch failure";
}

} // extern "C"

namespace bsl {

hipError_t launch_fwd_bf16(const Launch &a)
{
    fake::state().fwd_bf16++;
    fake::state().last_fwd = a;
    return fake::state().launch_result;
}

hipError_t launch_fwd_f32(const Launch &a)
{
    fake::state().fwd_f32++;
    fake::state().last_fwd = a;
    return fake::state().launch_result;
}

hipError_t launch_bwd_bf16(const BwdLaunch &a)
{
    fake::state().bwd_bf16++;
    fake::state().last_bwd = a;
    return fake::state().launch_result;
}

hipError_t launch_bwd_valu(const BwdLaunch &a, bool bf16)
{
    fake::state().bwd_valu++;
    fake::state().last_bwd = a;
    fake::state().last_bwd_valu_bf16 = bf16;
    return fake::state().launch_result;
}

int kmer_tiles(int32_t n_out) { return (n_out + 2047) / 2048; }

hipError_t launch_kmer(const KmerLaunch &a)
{
    fake::state().kmer++;
    fake::state().last_kmer = a;
    return fake::state().launch_result;
}

namespace {
float *g_scratch[8] = {};
}

hipError_t scratch_setup(int device)
{
    if (device < 0 || device > 7)
        return hipErrorInvalidDevice;
    if (!g_scratch[device]) {
        fake::state().scratch_lookups++;
        g_scratch[device] = fake::state().scratch;
    }
    return hipSuccess;
}

float *scratch_on(int device) { return device < 0 || device > 7 ? nullptr : g_scratch[device]; }

hipError_t launch_check(const int32_t *, int32_t, int32_t, int, int32_t *, hipStream_t)
{
    fake::state().check++;
    return fake::state().launch_result;
}

} // namespace bsl
