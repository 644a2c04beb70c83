// kmer.hip -- fused 2-bit k-mer tokenization, gfx950.
//
// Method: NucleoByte project page, section 2, item 1 ("Fused 2-Bit
// Tokenization": DNA text parsed on the GPU straight into packed integer IDs)
// and section 1 ("Token Blur": a fixed, bit-packed sliding window instead of a
// learned vocabulary); k-mer size and vocabulary from section 5 (6-mers, 4096
// IDs plus padding and mask entries).  A base is two bits, A = 0, C = 1, G = 2,
// T = 3, either case; the first base of a window is the most significant digit
// (the page's printed IDs, e.g. TGGGAC = 3745, fix this).  Window t of a
// sequence covers bases t .. t+k-1; a window holding any other byte is UNK.
//
// Mapping onto CDNA4 (the operation is a streaming pass: ~1 byte in, 4 bytes
// out per token, HBM-bound):
//  * one workgroup = one 2048-token tile of one output row; it stages the
//    tile's bytes (plus the k-1 bytes of overlap) in LDS with 16-byte loads from
//    16-byte aligned addresses, byte loads only where a chunk crosses either end
//    of the text buffer;
//  * each thread then takes 8 consecutive windows: it reads the 8 + k - 1 bytes
//    it needs as aligned LDS dwords, realigns them with v_alignbyte, computes
//    each base's code ((x >> 1) ^ (x >> 2)) & 3 -- the low bits of the ASCII
//    letters, case included -- and its validity, rolls the window ID along the
//    8 windows and writes them as two 16-byte stores -- streaming (non-
//    temporal) stores when the output is larger than half the Infinity Cache.
#include "kmer_launch.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int TPB = 256;            // threads per workgroup
constexpr int TPT = 8;              // windows per thread
constexpr int TILE = TPB * TPT;     // windows per workgroup
constexpr int STAGE_BYTES = TILE + 64;

// A, C, G, T in either case; anything else is not a base.  (x | 0x20) maps the
// four capitals onto their lower case; the lower-case letters a, c, g, t sit at
// offsets 0, 2, 6 and 19 from 'a'.
__device__ __forceinline__ bool is_base(uint32_t x)
{
    const uint32_t d = (x | 0x20u) - (uint32_t)'a';
    return d < 20u && ((0x80045u >> d) & 1u);
}

__device__ __forceinline__ uint32_t base_code(uint32_t x) { return ((x >> 1) ^ (x >> 2)) & 3u; }

template <int K, bool STREAM>
__global__ void __launch_bounds__(TPB) kmer_kernel(KmerLaunch a, int tiles)
{
    __shared__ __attribute__((aligned(16))) uint32_t stage[STAGE_BYTES / 4];
    const int tid = threadIdx.x;
    const int b = blockIdx.x / tiles, tile = blockIdx.x % tiles;
    const int32_t pad = 1 << (2 * K), unk = pad + 2;
    const uint32_t mask = (uint32_t)pad - 1u;

    // sequence b's bytes, clamped into the buffer
    int64_t s0 = a.starts[b], s1 = a.starts[b + 1];
    s0 = s0 < 0 ? 0 : (s0 > a.nbytes ? a.nbytes : s0);
    s1 = s1 < s0 ? s0 : (s1 > a.nbytes ? a.nbytes : s1);
    int64_t nt = s1 - s0 - K + 1;
    nt = nt < 0 ? 0 : (nt > a.n_out ? a.n_out : nt);
    if (tile == 0 && tid == 0 && a.ntok)
        a.ntok[b] = (int32_t)nt;

    const int t0 = tile * TILE;
    const int valid_end = (int)(nt < (int64_t)t0 + TILE ? nt : (int64_t)t0 + TILE);
    const uint8_t *buf = a.bases;
    const uintptr_t lo = (uintptr_t)buf, hi = lo + (uintptr_t)a.nbytes;
    const uintptr_t first = (uintptr_t)(buf + s0 + t0);
    const uintptr_t a_lo = first & ~(uintptr_t)15;
    const int shift = (int)(first - a_lo);

    if (valid_end > t0) {
        const int need = shift + (valid_end - t0) + K - 1;
        const int chunks = (need + 15) >> 4;
        for (int c = tid; c < chunks; c += TPB) {
            const uintptr_t addr = a_lo + (uintptr_t)c * 16u;
            u32x4 w;
            if (addr >= lo && addr + 16u <= hi) {
                w = *(const u32x4 *)addr;
            } else {
                uint32_t by[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const uintptr_t ai = addr + (uintptr_t)i;
                    by[i] = (ai >= lo && ai < hi) ? (uint32_t) * (const uint8_t *)ai : 0u;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    w[i] = by[4 * i] | (by[4 * i + 1] << 8) | (by[4 * i + 2] << 16) | (by[4 * i + 3] << 24);
            }
            *(u32x4 *)(stage + 4 * c) = w;
        }
        __syncthreads();
    }

    // eight consecutive windows per thread
    const int j0 = t0 + tid * TPT;
    if (j0 >= a.n_out)
        return;
    int32_t id[TPT];
    if (j0 < valid_end) {
        constexpr int NB = TPT + K - 1; // bases the eight windows cover
        const int o0 = shift + tid * TPT;
        const int wq = o0 >> 2, r = o0 & 3;
        uint32_t w[(NB + 3) / 4 + 2];
#pragma unroll
        for (int i = 0; i < (NB + 3) / 4 + 2; ++i)
            w[i] = stage[wq + i];
        uint32_t u[(NB + 3) / 4 + 1];
#pragma unroll
        for (int i = 0; i < (NB + 3) / 4 + 1; ++i)
            u[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], (uint32_t)r);
        uint32_t code[NB];
        int lastbad = -1; // position of the last non-base among bases 0 .. p
        uint32_t run = 0;
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            const uint32_t x = (u[p >> 2] >> (8 * (p & 3))) & 0xffu;
            code[p] = base_code(x);
            lastbad = is_base(x) ? lastbad : p;
            run = ((run << 2) | code[p]) & mask;
            if (p >= K - 1) {
                const int j = p - (K - 1);
                id[j] = lastbad >= j ? unk : (int32_t)run;
            }
        }
#pragma unroll
        for (int j = 0; j < TPT; ++j)
            if (j0 + j >= valid_end)
                id[j] = pad;
    } else {
#pragma unroll
        for (int j = 0; j < TPT; ++j)
            id[j] = pad;
    }
    int32_t *row = a.ids + (int64_t)b * a.n_out;
    if (j0 + TPT <= a.n_out && (((uintptr_t)(row + j0)) & 15u) == 0) {
        const i32x4 lo4 = {id[0], id[1], id[2], id[3]}, hi4 = {id[4], id[5], id[6], id[7]};
        if (STREAM) {
            // streaming stores: an output too large for the last-level cache
            // would only evict the text from it
            __builtin_nontemporal_store(lo4, (i32x4 *)(row + j0));
            __builtin_nontemporal_store(hi4, (i32x4 *)(row + j0 + 4));
        } else {
            *(i32x4 *)(row + j0) = lo4;
            *(i32x4 *)(row + j0 + 4) = hi4;
        }
    } else {
#pragma unroll
        for (int j = 0; j < TPT; ++j)
            if (j0 + j < a.n_out)
                row[j0 + j] = id[j];
    }
}

// Outputs past this size leave with streaming stores (MI355X's last-level
// cache, the Infinity Cache, holds 256 MB; a smaller output stays there for the
// embedding lookup that reads it next).
constexpr size_t STREAM_BYTES = (size_t)128 << 20;

template <int K>
hipError_t launch_k(const KmerLaunch &a, int tiles)
{
    const bool stream = (size_t)a.batch * (size_t)a.n_out * 4u > STREAM_BYTES;
    if (stream)
        hipLaunchKernelGGL((kmer_kernel<K, true>), dim3(a.batch * tiles), dim3(TPB), 0, a.stream, a,
                           tiles);
    else
        hipLaunchKernelGGL((kmer_kernel<K, false>), dim3(a.batch * tiles), dim3(TPB), 0, a.stream,
                           a, tiles);
    return hipGetLastError();
}

} // namespace

int kmer_tiles(int32_t n_out) { return (n_out + TILE - 1) / TILE; }

hipError_t launch_kmer(const KmerLaunch &a)
{
    const int tiles = a.n_out > 0 ? kmer_tiles(a.n_out) : 1; // one per row still writes ntok
    switch (a.k) {
    case 1: return launch_k<1>(a, tiles);
    case 2: return launch_k<2>(a, tiles);
    case 3: return launch_k<3>(a, tiles);
    case 4: return launch_k<4>(a, tiles);
    case 5: return launch_k<5>(a, tiles);
    case 6: return launch_k<6>(a, tiles);
    case 7: return launch_k<7>(a, tiles);
    case 8: return launch_k<8>(a, tiles);
    case 9: return launch_k<9>(a, tiles);
    case 10: return launch_k<10>(a, tiles);
    case 11: return launch_k<11>(a, tiles);
    case 12: return launch_k<12>(a, tiles);
    default: return hipErrorInvalidValue;
    }
}

} // namespace bsl
