// kmer_launch.h -- what the C-ABI layer hands to the tokenizer launcher (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {

// One k-mer tokenization call, after argument validation.
struct KmerLaunch {
    const uint8_t *bases;
    int64_t nbytes;
    const int64_t *starts; // device, batch + 1
    int32_t *ids;          // device, [batch][n_out]
    int32_t *ntok;         // device, [batch], or nullptr
    int32_t batch, k, n_out;
    hipStream_t stream;
};

int kmer_tiles(int32_t n_out);
hipError_t launch_kmer(const KmerLaunch &a);

} // namespace bsl
