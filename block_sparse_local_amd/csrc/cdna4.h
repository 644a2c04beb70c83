// cdna4.h -- small building blocks shared by the gfx950 kernels (internal).
//
// Types for MFMA operands, the 32x32 accumulator's row order, explicit memory
// waits, a barrier that does not drain outstanding loads, and the transposing
// LDS read.  Everything is in an anonymous namespace: each kernel source gets
// its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BLK = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Hardware hands workgroups to the 8 XCDs round robin.  Give XCD x the
// contiguous logical range [start_x, start_x + count_x) so its L2 sees
// neighbouring groups.  A bijection on [0, total).
__device__ __forceinline__ int xcd_contiguous(int g, int total)
{
    const int per = total / 8, extra = total % 8;
    const int x = g % 8, k = g / 8;
    return (x < extra ? x * (per + 1) : extra * (per + 1) + (x - extra) * per) + k;
}

// Key held by accumulator register r in lane half `half` of a 32x32 MFMA
// result: rows 8*(r/4) + 4*half + (r%4).
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// vmcnt(n) together with lgkmcnt(0); expcnt left alone.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void workgroup_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// The V^T operands of one 32-wide output tile: four transposing LDS reads at
// rows +0, +8, +16, +24 from `addr` (a 32-bit LDS address), waited for inside
// the same asm block.  The builtin form of this read makes the compiler drain
// every outstanding direct-to-LDS load first, which would empty the K/V ring on
// every step; issued here, nothing of these reads is left in flight.
template <int ROW_BYTES>
__device__ __forceinline__ void tr_tile(uint32_t addr, u32x2 &a0, u32x2 &a1, u32x2 &a2, u32x2 &a3)
{
    __asm__ volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                     "ds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
                     "ds_read_b64_tr_b16 %2, %4 offset:%6\n\t"
                     "ds_read_b64_tr_b16 %3, %4 offset:%7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
                     : "v"(addr), "i"(8 * ROW_BYTES), "i"(16 * ROW_BYTES), "i"(24 * ROW_BYTES));
}

// Like tr_tile, for tiles whose swizzle differs between rows r and r + 8 but
// repeats every 16 rows: reads rows r (a_r0), r + 8 (a_r8), r + 16 and r + 24.
template <int ROW_BYTES>
__device__ __forceinline__ void tr_tile_2a(uint32_t a_r0, uint32_t a_r8, u32x2 &a0, u32x2 &a1,
                                           u32x2 &a2, u32x2 &a3)
{
    __asm__ volatile("ds_read_b64_tr_b16 %0, %4\n\t"
                     "ds_read_b64_tr_b16 %1, %5\n\t"
                     "ds_read_b64_tr_b16 %2, %4 offset:%6\n\t"
                     "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3)
                     : "v"(a_r0), "v"(a_r8), "i"(16 * ROW_BYTES));
}

} // namespace
} // namespace bsl
