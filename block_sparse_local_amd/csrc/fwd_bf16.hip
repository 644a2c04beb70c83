// fwd_bf16.hip -- banded block-sparse attention forward, bf16 in/out, gfx950.
//
// Method: NucleoByte project page, section 3.  "Localized Block-Sparse
// Attention Matrix" fixes the work: with B = 32, query block i scores key blocks
// j with |i - j| <= R.  "Softmax Normalization & Online Numerical Stability"
// fixes the arithmetic: S = Q K^T / sqrt(d_k), and a running row maximum m, a
// running denominator l and a running output O are carried across the key
// blocks; O / l after the last block is the result.  Section 2, item 2
// ("Dynamic Ceiling Hardware Alignment") is why sequences arrive padded to a
// multiple of 32 with per-sequence lengths: keys past the length are masked,
// and blocks holding only padding are never visited.
//
// Mapping onto CDNA4:
//  * One workgroup = MQ waves = MQ consecutive query blocks of one (batch, head).
//    The workgroup sweeps the union of their bands, one key block per step; each
//    K/V block is brought into LDS once and serves every wave whose band covers
//    it (up to 2R+1 of them).  Two LDS buffers: block j+1 is fetched from HBM
//    into registers while block j is computed, then written to the other buffer.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    in the 32x32 accumulator each lane then owns one query (column) and 16 of
//    the 32 keys, so the row maximum is 15 in-register max ops plus one exchange
//    with the lane 32 away, and m, l and the rescale factor stay per lane.
//  * The output is also formed transposed, O^T += V^T P^T, so P^T is used as the
//    MFMA B operand straight from the score accumulator (rounded to bf16); the
//    key order inside the contraction is permuted to match the accumulator's
//    register order, and V is written into LDS transposed in that same order.
//  * exp is the hardware 2^x with log2(e) folded into the score scale.  The
//    running maximum is only moved when a row's maximum grows by more than 2^8;
//    O / l is unchanged by the choice of reference point, and p stays <= 256.
//  * l is summed from the same bf16-rounded probabilities the PV product uses.
//  * Padded keys of the last block are masked by select (never by a multiply)
//    and their V rows are zeroed as they enter LDS, so NaN padding cannot leak.
//  * Workgroup ids are remapped so that each XCD (its own L2) works through a
//    contiguous run of query groups: neighbouring groups share K/V halo blocks.
#include "launch.h"

#include <math.h>

namespace bsl {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BLK = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr float RESCALE_SLACK = 8.0f; // in log2 units

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    const int32_t *seqlens;
    float *lse;
    int32_t *active;
    uint32_t *masks;
    int32_t heads, n, nblk, ngroups, radius, total;
    float c; // scale * log2(e)
};

// Hardware hands workgroups to the 8 XCDs round robin.  Give XCD x the
// contiguous logical range [start_x, start_x + count_x) so its L2 sees
// neighbouring query groups.  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int g, int total)
{
    const int per = total / 8, extra = total % 8;
    const int x = g % 8, k = g / 8;
    return (x < extra ? x * (per + 1) : extra * (per + 1) + (x - extra) * per) + k;
}

// Key held by accumulator register r in lane half `half` of a 32x32 MFMA
// result: rows 8*(r/4) + 4*half + (r%4).
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Position of key kk inside a transposed V row in LDS: bits 2 and 3 swapped, so
// the 8 keys a lane half needs for one 16-key MFMA step are contiguous.
__device__ __forceinline__ int vt_pos(int kk)
{
    return (kk & ~12) | (((kk >> 2) & 1) << 3) | (((kk >> 3) & 1) << 2);
}

// Element offset of (dim row, key position) in the transposed V tile: rows of
// 32 bf16, 16-byte chunks XOR-swizzled by the row to spread LDS banks.
__device__ __forceinline__ int vt_off(int row, int pos)
{
    return row * BLK + ((((pos >> 3) ^ ((row >> 1) & 3))) << 3) + (pos & 7);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

template <int D, int MQ, bool CAUSAL, bool TRACE>
__global__ void __launch_bounds__(MQ * 64) fwd_bf16_kernel(Params p)
{
    constexpr int NT = MQ * 64;
    constexpr int KROW = D + 8;         // K row pitch in LDS (bf16): 16 bytes of pad
    constexpr int KSZ = BLK * KROW;     // K tile (bf16 elements)
    constexpr int VSZ = D * BLK;        // V^T tile: D rows of 32 keys
    constexpr int BUF = KSZ + VSZ;
    constexpr int NMT = D / 32;         // 32-wide output tiles
    constexpr int NKS = D / 16;         // 16-deep steps of the score contraction
    constexpr int KCH = BLK * D / 8;    // 16-byte chunks in a K block
    constexpr int KPT = (KCH + NT - 1) / NT;
    constexpr int VTASK = 16 * (D / 8); // (key pair, 8-dim chunk) tasks per V block
    constexpr int VPT = (VTASK + NT - 1) / NT;
    static_assert(D % 32 == 0 && D <= 128, "head_dim must be 32, 64 or 128");

    __shared__ __attribute__((aligned(16))) uint16_t lds[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;

    const int g = xcd_remap((int)blockIdx.x, p.total);
    const int grp = g % p.ngroups;
    const int bh = g / p.ngroups;
    const int b = bh / p.heads, h = bh % p.heads;
    int len = p.seqlens ? p.seqlens[b] : p.n;
    len = len < 0 ? 0 : (len > p.n ? p.n : len);
    const int nb = (len + BLK - 1) / BLK;
    const int R = p.radius, W = 2 * R + 1;
    const int i0 = grp * MQ;
    const int i = i0 + wave;
    const bool exists = i < p.nblk;
    const bool trace_here = TRACE && h == 0;

    const size_t base = (size_t)bh * (size_t)p.n * D;
    const uint16_t *qg = p.q + base;
    const uint16_t *kg = p.k + base;
    const uint16_t *vg = p.v + base;
    uint16_t *og = p.o + base;
    const size_t trace_row = ((size_t)b * p.nblk + (size_t)i) * (size_t)W;

    // ------------------------------------------------ blocks of pure padding
    if (i0 >= nb) {
        if (exists) {
            uint16_t *ob = og + (size_t)i * BLK * D;
            for (int c = lane; c < BLK * D / 8; c += 64)
                *(u32x4 *)(ob + (size_t)c * 8) = u32x4{0, 0, 0, 0};
            if (p.lse && half == 0)
                p.lse[(size_t)bh * p.n + (size_t)i * BLK + col] = -INFINITY;
            if (trace_here) {
                for (int s = lane; s < W; s += 64)
                    p.active[trace_row + s] = -1;
                for (int s = 0; s < W; ++s)
                    if (half == 0)
                        p.masks[(trace_row + s) * BLK + col] = 0u;
            }
        }
        return;
    }

    // -------------------------------------------------- key-block ranges
    int lo_w = 1, hi_w = 0; // this wave's band (empty unless i is a real block)
    if (exists && i < nb) {
        lo_w = i - R < 0 ? 0 : i - R;
        hi_w = i + R > nb - 1 ? nb - 1 : i + R;
        if (CAUSAL && hi_w > i)
            hi_w = i;
    }
    const int jlo = i0 - R < 0 ? 0 : i0 - R;
    int jhi = i0 + MQ - 1 + R > nb - 1 ? nb - 1 : i0 + MQ - 1 + R;
    if (CAUSAL && jhi > i0 + MQ - 1)
        jhi = i0 + MQ - 1;

    // ----------------------------------------------------------- Q fragment
    const int qrow = i * BLK + col;
    const bool qvalid = exists && qrow < len;
    bf16x8 qf[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        u32x4 x = u32x4{0, 0, 0, 0};
        if (qvalid)
            x = *(const u32x4 *)(qg + (size_t)qrow * D + s * 16 + half * 8);
        qf[s] = as_bf16x8(x);
    }

    f32x16 oacc[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            oacc[m][r] = 0.0f;
    float m_used = -INFINITY; // reference maximum (log2 units)
    float lsum = 0.0f;        // this lane's share of the denominator

    // --------------------------------------------------------- K/V staging
    u32x4 kreg[KPT];
    u32x4 vreg[VPT][2];
    auto fetch = [&](int j) {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int c = tid + u * NT;
            if (KCH % NT == 0 || c < KCH) {
                const int row = c / (D / 8), c8 = c % (D / 8);
                kreg[u] = *(const u32x4 *)(kg + (size_t)(j * BLK + row) * D + c8 * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int t = tid + u * NT;
            if (VTASK % NT == 0 || t < VTASK) {
                const int kp = t % 16, c8 = t / 16;
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int krow = j * BLK + 2 * kp + e;
                    u32x4 x = *(const u32x4 *)(vg + (size_t)krow * D + c8 * 8);
                    // padded keys: zero V so that p = 0 never meets a NaN
                    vreg[u][e] = krow < len ? x : u32x4{0, 0, 0, 0};
                }
            }
        }
    };
    auto deposit = [&](int buf) {
        uint16_t *kl = lds + buf * BUF;
        uint16_t *vt = kl + KSZ;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int c = tid + u * NT;
            if (KCH % NT == 0 || c < KCH) {
                const int row = c / (D / 8), c8 = c % (D / 8);
                *(u32x4 *)(kl + row * KROW + c8 * 8) = kreg[u];
            }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int t = tid + u * NT;
            if (VTASK % NT == 0 || t < VTASK) {
                const int kp = t % 16, c8 = t / 16;
                const int pos = vt_pos(2 * kp);
                const u32x4 a = vreg[u][0], bb = vreg[u][1];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t even = (a[w] & 0xFFFFu) | (bb[w] << 16);
                    const uint32_t odd = (a[w] >> 16) | (bb[w] & 0xFFFF0000u);
                    const int row = c8 * 8 + 2 * w;
                    *(uint32_t *)(vt + vt_off(row, pos)) = even;
                    *(uint32_t *)(vt + vt_off(row + 1, pos)) = odd;
                }
            }
        }
    };

    fetch(jlo);
    deposit(0);
    __syncthreads();

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    for (int j = jlo; j <= jhi; ++j) {
        const int cur = (j - jlo) & 1;
        const bool more = j < jhi;
        if (more)
            fetch(j + 1);

        if (j >= lo_w && j <= hi_w) {
            const uint16_t *kl = lds + cur * BUF;
            const uint16_t *vt = kl + KSZ;

            // S^T = K_j Q_i^T  (rows: keys, columns: queries)
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 a = as_bf16x8(*(const u32x4 *)(kl + col * KROW + ks * 16 + half * 8));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
            }

            // padding and causal masks: only the last real block and the diagonal
            const bool need_mask = (j == nb - 1 && (len & (BLK - 1)) != 0) || (CAUSAL && j == i);
            uint32_t part = 0;
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j * BLK + acc_row(r, half);
                    const bool keep = key < len && (!CAUSAL || key <= qrow);
                    s[r] = keep ? s[r] : -INFINITY;
                    if (TRACE)
                        part |= (keep ? 1u : 0u) << acc_row(r, half);
                }
            }
            if (trace_here) {
                uint32_t word = need_mask ? (part | (uint32_t)__shfl_xor((int)part, 32)) : 0xFFFFFFFFu;
                if (!qvalid)
                    word = 0u;
                const size_t slot = trace_row + (size_t)(j - lo_w);
                if (half == 0)
                    p.masks[slot * BLK + col] = word;
                if (lane == 0)
                    p.active[slot] = j;
            }

            // running maximum (log2 units), moved only when it grows a lot
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                mx = fmaxf(mx, s[r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = mx * p.c;
            if (__ballot(mt > m_used + RESCALE_SLACK) != 0) {
                const float mn = fmaxf(m_used, mt);
                const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
#pragma unroll
                for (int m = 0; m < NMT; ++m)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        oacc[m][r] *= alpha;
                lsum *= alpha;
                m_used = mn;
            }

            // probabilities, rounded once to bf16 for both l and P V
            uint32_t pk[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float e0 = __builtin_amdgcn_exp2f(fmaf(s[2 * u], p.c, -m_used));
                const float e1 = __builtin_amdgcn_exp2f(fmaf(s[2 * u + 1], p.c, -m_used));
                const bf16x2 pr = __builtin_convertvector(f32x2{e0, e1}, bf16x2);
                lsum = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum, false);
                pk[u] = __builtin_bit_cast(uint32_t, pr);
            }
            const bf16x8 pb0 = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
            const bf16x8 pb1 = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});

            // O^T += V_j^T P^T
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const int row = m * 32 + col;
                const bf16x8 a0 = as_bf16x8(*(const u32x4 *)(vt + vt_off(row, half * 8)));
                const bf16x8 a1 = as_bf16x8(*(const u32x4 *)(vt + vt_off(row, 16 + half * 8)));
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pb0, oacc[m], 0, 0, 0);
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pb1, oacc[m], 0, 0, 0);
            }
        }

        if (more)
            deposit(cur ^ 1);
        __syncthreads();
    }

    // ------------------------------------------------------------- finalize
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (!exists)
        return;
    const float inv = qvalid ? 1.0f / lt : 0.0f;
    uint16_t *orow = og + (size_t)qrow * D;
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x2 lo2 = {oacc[m][4 * a] * inv, oacc[m][4 * a + 1] * inv};
            f32x2 hi2 = {oacc[m][4 * a + 2] * inv, oacc[m][4 * a + 3] * inv};
            if (!qvalid) {
                lo2 = f32x2{0.0f, 0.0f};
                hi2 = f32x2{0.0f, 0.0f};
            }
            const u32x2 packed = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, bf16x2)),
                                  __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2))};
            *(u32x2 *)(orow + m * 32 + 8 * a + 4 * half) = packed;
        }
    }
    if (p.lse && half == 0)
        p.lse[(size_t)bh * p.n + (size_t)qrow] =
            qvalid ? (m_used + __builtin_amdgcn_logf(lt)) * LN2 : -INFINITY;
    if (trace_here) {
        const int used = hi_w >= lo_w ? hi_w - lo_w + 1 : 0;
        for (int s = used + lane; s < W; s += 64)
            p.active[trace_row + s] = -1;
        for (int s = used; s < W; ++s)
            if (half == 0)
                p.masks[(trace_row + s) * BLK + col] = 0u;
    }
}

template <int D, int MQ, bool CAUSAL, bool TRACE>
hipError_t launch_t(const Launch &a, const Params &p)
{
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MQ, CAUSAL, TRACE>), dim3(p.total), dim3(MQ * 64), 0,
                       a.stream, p);
    return hipGetLastError();
}

template <int D, int MQ>
hipError_t launch_d(const Launch &a, const Params &p)
{
    const bool tr = a.active != nullptr;
    if (a.causal)
        return tr ? launch_t<D, MQ, true, true>(a, p) : launch_t<D, MQ, true, false>(a, p);
    return tr ? launch_t<D, MQ, false, true>(a, p) : launch_t<D, MQ, false, false>(a, p);
}

} // namespace

hipError_t launch_fwd_bf16(const Launch &a)
{
    constexpr int MQ = 4;
    Params p;
    p.q = (const uint16_t *)a.q;
    p.k = (const uint16_t *)a.k;
    p.v = (const uint16_t *)a.v;
    p.o = (uint16_t *)a.o;
    p.seqlens = a.seqlens;
    p.lse = a.lse;
    p.active = a.active;
    p.masks = a.masks;
    p.heads = a.heads;
    p.n = a.n;
    p.nblk = a.n / BLK;
    p.ngroups = (p.nblk + MQ - 1) / MQ;
    p.radius = a.radius;
    p.total = a.batch * a.heads * p.ngroups;
    p.c = a.scale * LOG2E;
    switch (a.head_dim) {
    case 32: return launch_d<32, MQ>(a, p);
    case 64: return launch_d<64, MQ>(a, p);
    case 128: return launch_d<128, MQ>(a, p);
    default: return hipErrorInvalidValue;
    }
}

} // namespace bsl
