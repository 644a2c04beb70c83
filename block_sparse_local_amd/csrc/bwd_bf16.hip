// bwd_bf16.hip -- backward pass of the banded block-sparse attention, bf16, gfx950.
//
// Method: NucleoByte project page, section 3, "Custom Backpropagation": with P
// the forward's softmax, a per-row correction D_t = sum_c dO_tc O_tc and
// dS_ts = P_ts (dO_t . V_s - D_t).  The gradients then follow by the chain
// rule through S = scale Q K^T and O = P V:
//     dV = P^T dO,   dQ = scale dS K,   dK = scale dS^T Q.
// The band, padding and causal rules are the forward's (section 3, "Localized
// Block-Sparse Attention Matrix"; section 2, item 2).  P is recomputed from the
// scores and the forward's stored log-sum-exp: P = exp(S - lse).
//
// Two kernels, in stream order:
//  * dq: one wave per query block, 4 per workgroup, sweeping the union of their
//    key bands like the forward (ring of K/V blocks filled by direct-to-LDS
//    loads, rotated sweep, XCD-contiguous groups).  First D_t in fp32 from the
//    bf16 dO fragments the wave holds anyway and the same elements of O (0 on
//    padded rows), written out for dkv.  Then per key block
//        S^T = K Q^T,  dP^T = V dO^T,  P^T = 2^(S^T c - lse log2 e),
//        dS^T = P^T (dP^T - D),  dQ^T += K^T dS^T.
//    As in the forward each lane owns one query column, so lse and D are
//    per-lane scalars; dS^T enters the last product as the MFMA B operand
//    straight from the accumulator, and K^T comes from transposing LDS reads.
//  * dkv: one wave per key block, 4 per workgroup, sweeping the union of their
//    query bands (ring of Q, dO, lse and D blocks).  Per query block
//        S = Q K^T,  dP = dO V^T  (each lane owns one key column),
//        dV^T += dO^T P,  dK^T += Q^T dS.
//    K stays in registers; the wave's V block waits in LDS, which is what
//    lets the two fp32 accumulators and everything else fit 256 registers at
//    d 128 (two waves per SIMD) and 168 at d 64 (three).
// P and dS are rounded once to bf16 for the MFMAs; every sum is fp32.  K (in
// dq) and Q, dO (in dkv) are read both row-wise and transposed, so their LDS
// tiles use one swizzle that keeps both access patterns free of bank
// conflicts.  Masks are applied by select, and rows past a sequence's end are
// zeroed in LDS before any transposing read, so NaN padding cannot leak through
// a zero probability.
#include "cdna4.h"
#include "bwd_launch.h"

#include <math.h>

namespace bsl {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS tile of 32 rows x D bf16 for the backward kernels: row-major, 16-byte
// chunk c of row r at chunk position c ^ swz(r).  Row reads take one chunk from
// 16 consecutive rows; transposing reads take 4 consecutive rows x 4 chunks.
// swz gives 16 consecutive rows 16 distinct positions (one per bank group of a
// 256-byte window) and sends 4 consecutive rows to 4 different aligned 4-chunk
// sets.  swz(r + 16) == swz(r) and swz(r + 8) == swz(r) ^ 2.
template <int D>
struct BTile {
    static_assert(D == 64 || D == 128, "head_dim 64 or 128");
    static constexpr int CPR = D / 8;
    static constexpr int BYTES = BLK * D * 2;
    static constexpr int ROW_BYTES = D * 2;
    __device__ static __forceinline__ int swz(int r)
    {
        if constexpr (D == 128)
            return ((r & 3) << 2) | ((r >> 2) & 3);
        else // two rows share a 256-byte window: swizzle by the row pair m = r / 2
            return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    }
};

struct BParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;
    const int32_t *seqlens; // padded layout: lengths (or nullptr)
    const int32_t *cu;      // packed layout: sequence start offsets, batch + 1 of them
    int32_t tokens;         // packed layout: rows in the buffers
    uint16_t *dq, *dk, *dv;
    float *delta;
    int32_t heads, n, nblk, ngroups, radius, total;
    int32_t window; // 0: the block band; >= 1: keys within this many tokens
    float c;     // scale * log2(e)
    float scale; // scale
};

// Where sequence b's rows of head h live and how many are real.  Padded layout
// [batch][heads][n][D]: rows D apart; lse and delta [batch][heads][n].  Packed
// layout [tokens][heads][D]: rows heads D apart from (cu[b] heads + h) D; lse
// and delta [heads][tokens].  Offsets read from the device are clamped so that
// every row index below stays inside the buffers whatever they hold.
template <int D, bool VARLEN>
struct BSeq {
    size_t base, lbase, rs;
    int len;
    __device__ __forceinline__ BSeq(const BParams &p, int b, int h)
    {
        if (VARLEN) {
            int s0 = p.cu[b], s1 = p.cu[b + 1];
            s0 = s0 < 0 ? 0 : (s0 > p.tokens ? p.tokens : s0);
            s1 = s1 < s0 ? s0 : (s1 > p.tokens ? p.tokens : s1);
            len = s1 - s0 > p.n ? p.n : s1 - s0;
            base = ((size_t)s0 * (size_t)p.heads + (size_t)h) * D;
            lbase = (size_t)h * (size_t)p.tokens + (size_t)s0;
            rs = (size_t)p.heads * D;
        } else {
            len = p.seqlens ? p.seqlens[b] : p.n;
            len = len < 0 ? 0 : (len > p.n ? p.n : len);
            base = ((size_t)b * p.heads + h) * (size_t)p.n * D;
            lbase = ((size_t)b * p.heads + h) * (size_t)p.n;
            rs = D;
        }
    }
};

// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle, no index stride).
constexpr int BUFFER_WORD3 = 0x00020000;

// ------------------------------------------------------------ shared parts
// Band of block x (a query block for dq, a key block for dkv) within nb real
// blocks: the blocks it pairs with.  For dq the partners are key blocks <= x
// when causal; for dkv they are query blocks >= x.
__device__ __forceinline__ void band_of(int x, int nb, int R, bool causal, bool partners_below,
                                        int &lo, int &hi)
{
    lo = x - R < 0 ? 0 : x - R;
    hi = x + R > nb - 1 ? nb - 1 : x + R;
    if (causal) {
        if (partners_below)
            hi = hi > x ? x : hi;
        else
            lo = lo < x ? x : lo;
    }
}

// Fill slot range of one 16 KB-or-8 KB tile pair in a ring stage: slot s of
// the stage (16 bytes at stage + 16 s) holds tile A (s < SLOTS/2) or tile B.
// Buffer loads into LDS: a scalar buffer resource based at the block's first
// row of each tile (bounds-checked against the block) plus a per-lane offset
// that does not depend on the block, so no vector ALU goes into addresses.
// Rows are rs elements apart; rows past `last` (the block's last row inside the
// sequence, packed layout) repeat it, so no load leaves the sequence; their
// values are zeroed or masked before use.
template <int D, int NT, int LPT, bool VARLEN>
__device__ __forceinline__ void issue_pair(uint8_t *stage, const uint16_t *ga, const uint16_t *gb,
                                          int row0, size_t rs, int last, int tid, int wave)
{
    using T = BTile<D>;
    constexpr int SLOTS = 2 * T::BYTES / 16;
    const int bytes = (int)((size_t)(last + 1) * rs * 2);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(ga + (size_t)row0 * rs), (short)0, bytes, BUFFER_WORD3);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(gb + (size_t)row0 * rs), (short)0, bytes, BUFFER_WORD3);
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
        const int s = u * NT + tid;
        const bool second = u * NT + wave * 64 >= SLOTS / 2; // uniform per wave
        const int t = second ? s - SLOTS / 2 : s;
        const int r = t / T::CPR, cp = t % T::CPR;
        const int c = cp ^ T::swz(r);
        const int rr = VARLEN && r > last ? last : r;
        const uint32_t off = (uint32_t)((size_t)rr * rs + (size_t)c * 8) * 2u;
        uint8_t *dst = stage + (u * NT + wave * 64) * 16;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? rb : ra, (lds_void *)dst, 16, off, 0, 0, 0);
    }
}

// Zero rows [r0, 32) of an LDS tile (whole rows: the swizzle does not matter).
template <int D, int NT>
__device__ __forceinline__ void zero_tail_rows(uint8_t *tile, int r0, int tid)
{
    using T = BTile<D>;
    for (int x = tid; x < (BLK - r0) * T::CPR; x += NT)
        *(u32x4 *)(tile + (r0 * T::CPR + x) * 16) = u32x4{0, 0, 0, 0};
}

// Row read of logical chunk `chunk` of row `row` (MFMA A operand fragment).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint8_t *tile, int row, int chunk)
{
    using T = BTile<D>;
    return as_bf16x8(*(const u32x4 *)(tile + row * T::ROW_BYTES + ((chunk ^ T::swz(row)) << 4)));
}

// The transposed operand of output tile m (32 columns of D) from an LDS tile:
// two MFMA A fragments (keys or queries 0-15 and 16-31 in the accumulator's
// permuted order).
template <int D>
__device__ __forceinline__ void tr_frags(const uint8_t *tile, int m, int tr_row, int tr_col,
                                         bf16x8 &a0, bf16x8 &a1)
{
    using T = BTile<D>;
    const int chunk = 4 * m + (tr_col >> 3);
    const uint32_t base = (uint32_t)(size_t)(lds_u8 *)tile + (tr_col & 7) * 2;
    const uint32_t a_r0 = base + tr_row * T::ROW_BYTES + ((chunk ^ T::swz(tr_row)) << 4);
    const uint32_t a_r8 = base + (tr_row + 8) * T::ROW_BYTES + ((chunk ^ T::swz(tr_row + 8)) << 4);
    u32x2 r0, r1, r2, r3;
    tr_tile_2a<T::ROW_BYTES>(a_r0, a_r8, r0, r1, r2, r3);
    const bf16x4 q0 = __builtin_bit_cast(bf16x4, r0), q1 = __builtin_bit_cast(bf16x4, r1);
    const bf16x4 q2 = __builtin_bit_cast(bf16x4, r2), q3 = __builtin_bit_cast(bf16x4, r3);
    a0 = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
    a1 = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Pack 16 fp32 accumulator values into the two bf16 B fragments of a product
// that contracts over the accumulator's rows.
__device__ __forceinline__ void pack_b(const float *x, bf16x8 &b0, bf16x8 &b1)
{
    uint32_t pk[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
        pk[u] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2 * u], x[2 * u + 1]}, bf16x2));
    b0 = as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]});
    b1 = as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]});
}

// Store a transposed fp32 accumulator (NMT tiles of 32 columns) as bf16 row
// `row` of `out` (already offset to the slice), scaled; zeros when !valid.
template <int NMT>
__device__ __forceinline__ void store_rowT(uint16_t *out_row, const f32x16 *acc, float mul, bool valid,
                                           int half, bool store = true)
{
    // lanes l and l + 32 hold the two 4-element halves of each 8-element run;
    // one exchange gives each lane two whole runs, stored 16 bytes at a time
    // (call with the whole wave active)
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        u32x2 pk4[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x2 lo2 = {acc[m][4 * a] * mul, acc[m][4 * a + 1] * mul};
            f32x2 hi2 = {acc[m][4 * a + 2] * mul, acc[m][4 * a + 3] * mul};
            if (!valid) {
                lo2 = f32x2{0.0f, 0.0f};
                hi2 = f32x2{0.0f, 0.0f};
            }
            pk4[a] = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, bf16x2)),
                           __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2))};
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const u32x2 mine = half ? pk4[2 * k + 1] : pk4[2 * k];
            const u32x2 give = half ? pk4[2 * k] : pk4[2 * k + 1];
            u32x2 got;
            got[0] = (uint32_t)__shfl_xor((int)give[0], 32);
            got[1] = (uint32_t)__shfl_xor((int)give[1], 32);
            const u32x4 run = half ? u32x4{got[0], got[1], mine[0], mine[1]}
                                   : u32x4{mine[0], mine[1], got[0], got[1]};
            if (store)
                *(u32x4 *)(out_row + m * 32 + 8 * (2 * k + half)) = run;
        }
    }
}

// ------------------------------------------------------------------- dq
template <int D, int NSTAGE, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) dq_kernel(BParams p)
{
    using T = BTile<D>;
    constexpr int MQ = 4, NT = 256;
    constexpr int NMT = D / 32, NKS = D / 16;
    constexpr int STAGE = 2 * T::BYTES; // K tile then V tile
    constexpr int LPT = STAGE / 16 / NT;
    static_assert(STAGE / 16 % NT == 0 && LPT >= 1, "slots split evenly over threads");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    const int g = xcd_contiguous((int)blockIdx.x, p.total);
    // packed layout with 128-byte head pieces (D 64): the heads of a group run
    // consecutively, so neighbouring workgroups read whole token rows
    constexpr bool HEADS_FASTEST = VARLEN && D * 2 < 256;
    const int bh = g / p.ngroups;
    const int grp = HEADS_FASTEST ? (g / p.heads) % p.ngroups : g % p.ngroups;
    const int b = HEADS_FASTEST ? g / p.heads / p.ngroups : bh / p.heads;
    const int h = HEADS_FASTEST ? g % p.heads : bh % p.heads;
    const BSeq<D, VARLEN> sq(p, b, h);
    const int len = sq.len;
    const int nb = (len + BLK - 1) / BLK;
    const int R = p.radius;
    const int i0 = grp * MQ, i = i0 + wave;
    // packed layout: rows past the sequence belong to the next one, so only
    // the sequence's own blocks exist; padded layout: every block of the buffer
    const bool exists = i < (VARLEN ? nb : p.nblk);
    const size_t base = sq.base, RS = sq.rs;
    const int qrow = i * BLK + col;
    const bool qvalid = exists && qrow < len;
    uint16_t *dq_row = p.dq + base + (size_t)qrow * RS;

    if (i0 >= nb) { // a group of padding only
        if (!VARLEN && exists) {
            for (int c = lane; c < BLK * D / 8; c += 64)
                *(u32x4 *)(p.dq + base + (size_t)i * BLK * D + (size_t)c * 8) = u32x4{0, 0, 0, 0};
            if (half == 0)
                p.delta[sq.lbase + qrow] = 0.0f;
        }
        return;
    }
    int lo_w = 1, hi_w = 0;
    if (exists && i < nb)
        band_of(i, nb, R, CAUSAL, true, lo_w, hi_w);
    const int jlo = i0 - R < 0 ? 0 : i0 - R;
    int jhi = i0 + MQ - 1 + R > nb - 1 ? nb - 1 : i0 + MQ - 1 + R;
    if (CAUSAL && jhi > i0 + MQ - 1)
        jhi = i0 + MQ - 1;
    const int L = jhi - jlo + 1;
    const int P = CAUSAL ? MQ + R : MQ + 2 * R;
    const int rot = L == P ? (P - jlo % P) % P : 0;
    auto block_at = [&](int t) {
        const int x = t + rot;
        return jlo + (x >= L ? x - L : x);
    };
    const uint16_t *const kg = p.k + base, *const vg = p.v + base;
    auto issue = [&](int j, int stage) {
        const int last = len - 1 - j * BLK < BLK - 1 ? len - 1 - j * BLK : BLK - 1;
        issue_pair<D, NT, LPT, VARLEN>(lds + stage * STAGE, kg, vg, j * BLK, RS,
                                       VARLEN ? last : BLK - 1, tid, wave);
    };

    // this wave's query and output-gradient fragments, its rows of O (for D)
    // and lse, all loaded at once and on every lane (a lane past the sequence
    // reads its first row, which exists, and zeroes what it read below), then
    // the ring's first stages, and only then the wait: one memory round trip
    // before the loop instead of one per dependent load
    const int qread = qvalid ? qrow : 0;
    bf16x8 qf[NKS], gf[NKS];
    u32x4 orow[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const size_t off = base + (size_t)qread * RS + s * 16 + half * 8;
        qf[s] = as_bf16x8(*(const u32x4 *)(p.q + off));
        gf[s] = as_bf16x8(*(const u32x4 *)(p.dout + off));
        orow[s] = *(const u32x4 *)(p.o + off);
    }
    const float lse_read = p.lse[sq.lbase + qread];
#pragma unroll
    for (int a = 0; a < NSTAGE - 1; ++a)
        if (a < L)
            issue(block_at(a), a);
    const float lse2 = qvalid ? lse_read * LOG2E : 0.0f;
    // D_t = sum_c dO_tc O_tc: this lane's half of the row (the dO fragments it
    // holds) against the same elements of O, then the other half from lane +- 32;
    // written for the key-stationary kernel, 0 on rows past the length
    float Dt = 0.0f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (!qvalid) {
            qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
            gf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
        }
        const bf16x8 ov = as_bf16x8(orow[s]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            Dt = fmaf((float)gf[s][e], (float)ov[e], Dt);
        __asm__ volatile("" : "+v"(qf[s]), "+v"(gf[s]));
    }
    Dt += __shfl_xor(Dt, 32);
    if ((VARLEN ? qvalid : exists) && half == 0)
        p.delta[sq.lbase + qrow] = Dt;

    f32x16 acc[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            acc[m][r] = 0.0f;

    const int grp16 = lane >> 4, li = lane & 15;
    const int tr_row = 4 * half + (li >> 2);
    const int tr_col = 16 * (grp16 & 1) + 4 * (li & 3);

    for (int t = 0; t < L; ++t) {
        const int j = block_at(t);
        const int stage = t % NSTAGE;
        if (t + NSTAGE - 2 < L)
            wait_vm_lgkm0<(NSTAGE - 2) * LPT>();
        else
            wait_vm_lgkm0<0>();
        workgroup_barrier();
        if (t + NSTAGE - 1 < L)
            issue(block_at(t + NSTAGE - 1), (t + NSTAGE - 1) % NSTAGE);
        uint8_t *kl = lds + stage * STAGE;
        const uint8_t *vl = kl + T::BYTES;
        const bool pad_block = j == nb - 1 && (len & (BLK - 1)) != 0;
        if (pad_block) {
            // K rows past the end enter the transposed product: make them 0
            zero_tail_rows<D, NT>(kl, len - j * BLK, tid);
            wait_vm_lgkm0<63>();
            workgroup_barrier();
        }
        if (j < lo_w || j > hi_w)
            continue;

        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.0f;
            dp[r] = 0.0f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 ka = row_frag<D>(kl, col, 2 * ks + half);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 va = row_frag<D>(vl, col, 2 * ks + half);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, gf[ks], dp, 0, 0, 0);
        }
        // Schedule the two products' operand reads four ahead of their MFMAs
        // (left alone, the compiler keeps one read in flight and every MFMA
        // waits out a full LDS round trip; the registers are there, since the
        // kernel runs two waves per SIMD at d 128 either way).
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0); // 4 LDS reads
#pragma unroll
        for (int x = 0; x < 2 * NKS - 4; ++x) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); // 1 LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0); // the last 4 MFMAs
        // a token window also cuts blocks whose farthest pair lies beyond it
        const int dj = j > i ? j - i : i - j;
        const bool need_mask = !qvalid || pad_block || (CAUSAL && j == i) ||
                               (p.window > 0 && dj * BLK + BLK - 1 > p.window);
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], p.c, -lse2));
            ds[r] = pr * (dp[r] - Dt);
        }
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = j * BLK + acc_row(r, half);
                const int dist = qrow > key ? qrow - key : key - qrow;
                const bool keep = qvalid && key < len && (!CAUSAL || key <= qrow) &&
                                  (p.window <= 0 || dist <= p.window);
                ds[r] = keep ? ds[r] : 0.0f;
            }
        }
        bf16x8 db0, db1;
        pack_b(ds, db0, db1);
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            bf16x8 a0, a1;
            tr_frags<D>(kl, m, tr_row, tr_col, a0, a1);
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, db0, acc[m], 0, 0, 0);
            acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, db1, acc[m], 0, 0, 0);
        }
    }
    if (exists)
        store_rowT<NMT>(dq_row, acc, p.scale, qvalid, half, !VARLEN || qvalid);
}

// ------------------------------------------------------------------ dkv
// Occupancy target: the register budget that gives two waves per SIMD at
// d 128 and three at d 64 (at d 128 the packed-layout instances spill two or
// three values, none of them inside the loop).
template <int D, int NSTAGE, bool CAUSAL, bool VARLEN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 3)))
dkv_kernel(BParams p)
{
    using T = BTile<D>;
    constexpr int MK = 4, NT = 256;
    constexpr int NMT = D / 32, NKS = D / 16;
    constexpr int TILES = 2 * T::BYTES;      // Q tile then dO tile
    constexpr int STAGE = TILES + 2 * BLK * 4; // then lse[32], D[32]
    constexpr int LPT = TILES / 16 / NT;
    static_assert(TILES / 16 % NT == 0 && LPT >= 1, "slots split evenly over threads");

    // the ring, then one V tile per wave
    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE + MK * T::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    const int g = xcd_contiguous((int)blockIdx.x, p.total);
    // packed layout with 128-byte head pieces (D 64): the heads of a group run
    // consecutively, so neighbouring workgroups read whole token rows
    constexpr bool HEADS_FASTEST = VARLEN && D * 2 < 256;
    const int bh = g / p.ngroups;
    const int grp = HEADS_FASTEST ? (g / p.heads) % p.ngroups : g % p.ngroups;
    const int b = HEADS_FASTEST ? g / p.heads / p.ngroups : bh / p.heads;
    const int h = HEADS_FASTEST ? g % p.heads : bh % p.heads;
    const BSeq<D, VARLEN> sq(p, b, h);
    const int len = sq.len;
    const int nb = (len + BLK - 1) / BLK;
    const int R = p.radius;
    const int j0 = grp * MK, j = j0 + wave;
    const bool exists = j < (VARLEN ? nb : p.nblk);
    const size_t base = sq.base, RS = sq.rs;
    const size_t rbase = sq.lbase; // lse, delta
    const int krow = j * BLK + col;
    const bool kvalid = exists && krow < len;
    uint16_t *dk_row = p.dk + base + (size_t)krow * RS;
    uint16_t *dv_row = p.dv + base + (size_t)krow * RS;

    if (j0 >= nb) {
        if (!VARLEN && exists)
            for (int c = lane; c < BLK * D / 8; c += 64) {
                const size_t off = base + (size_t)j * BLK * D + (size_t)c * 8;
                *(u32x4 *)(p.dk + off) = u32x4{0, 0, 0, 0};
                *(u32x4 *)(p.dv + off) = u32x4{0, 0, 0, 0};
            }
        return;
    }
    int lo_w = 1, hi_w = 0;
    if (exists && j < nb)
        band_of(j, nb, R, CAUSAL, false, lo_w, hi_w);
    const int ilo = CAUSAL ? j0 : (j0 - R < 0 ? 0 : j0 - R);
    const int ihi = j0 + MK - 1 + R > nb - 1 ? nb - 1 : j0 + MK - 1 + R;
    const int L = ihi - ilo + 1;
    const int P = CAUSAL ? MK + R : MK + 2 * R;
    const int rot = L == P ? (P - ilo % P) % P : 0;
    auto block_at = [&](int t) {
        const int x = t + rot;
        return ilo + (x >= L ? x - L : x);
    };
    // Q and dO tiles by every thread; lse (wave 0) and D (wave 1), 32 floats
    // each, by lanes 0-7, so waves 0 and 1 have one more load in flight per
    // stage.  All are buffer loads bounded by the block's rows inside the
    // sequence.
    const uint16_t *const qg = p.q + base, *const gg = p.dout + base;
    const float *const lg = p.lse + rbase, *const dg = p.delta + rbase;
    auto issue = [&](int i, int stage) {
        uint8_t *st = lds + stage * STAGE;
        const int last_in = len - 1 - i * BLK < BLK - 1 ? len - 1 - i * BLK : BLK - 1;
        const int last = VARLEN ? last_in : BLK - 1;
        issue_pair<D, NT, LPT, VARLEN>(st, qg, gg, i * BLK, RS, last, tid, wave);
        if (wave < 2 && lane < 8) {
            const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((wave == 0 ? lg : dg) + i * BLK), (short)0, (last + 1) * 4, BUFFER_WORD3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(st + TILES + wave * BLK * 4), 16,
                                                     (uint32_t)lane * 16u, 0, 0, 0);
        }
    };

    // this wave's key and value fragments (B operands of S = Q K^T, dP = dO V^T);
    // the value fragments go to the wave's own LDS tile, each lane writing the
    // chunks it reads back in the loop (so no other lane or wave is involved),
    // and the empty asm keeps the compiler from carrying them in registers.
    // Both are loaded on every lane (a lane past the sequence reads its first
    // row and zeroes it) before the ring's first stages are issued, so that
    // all of it costs one memory round trip rather than one per fragment.
    bf16x8 kf[NKS];
    u32x4 vrow[NKS];
    uint8_t *const vtile = lds + NSTAGE * STAGE + wave * T::BYTES;
    const int kread = kvalid ? krow : 0;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        const size_t off = base + (size_t)kread * RS + s * 16 + half * 8;
        kf[s] = as_bf16x8(*(const u32x4 *)(p.k + off));
        vrow[s] = *(const u32x4 *)(p.v + off);
    }
#pragma unroll
    for (int a = 0; a < NSTAGE - 1; ++a)
        if (a < L)
            issue(block_at(a), a);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (!kvalid) {
            kf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
            vrow[s] = u32x4{0, 0, 0, 0};
        }
        *(u32x4 *)(vtile + col * T::ROW_BYTES + (((2 * s + half) ^ T::swz(col)) << 4)) = vrow[s];
        __asm__ volatile("" : "+v"(kf[s]));
    }
    __asm__ volatile("" ::: "memory");

    f32x16 dka[NMT], dva[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            dka[m][r] = 0.0f;
            dva[m][r] = 0.0f;
        }

    const int grp16 = lane >> 4, li = lane & 15;
    const int tr_row = 4 * half + (li >> 2);
    const int tr_col = 16 * (grp16 & 1) + 4 * (li & 3);
    const float c = p.c;

    for (int t = 0; t < L; ++t) {
        const int i = block_at(t);
        const int stage = t % NSTAGE;
        if (t + NSTAGE - 2 < L) {
            if (wave < 2)
                wait_vm_lgkm0<(NSTAGE - 2) * (LPT + 1)>();
            else
                wait_vm_lgkm0<(NSTAGE - 2) * LPT>();
        } else {
            wait_vm_lgkm0<0>();
        }
        workgroup_barrier();
        if (t + NSTAGE - 1 < L)
            issue(block_at(t + NSTAGE - 1), (t + NSTAGE - 1) % NSTAGE);
        uint8_t *ql = lds + stage * STAGE;
        uint8_t *gl = ql + T::BYTES;
        // The V tile is addressed from the Q tile's lane addresses plus a
        // uniform offset that the compiler cannot see through, so that it does
        // not keep a second set of per-lane addresses live across the loop
        // (at d 128 that pushed other values out to scratch, and each reload
        // then waited for the ring's loads in flight).
        int voff = (int)(vtile - ql);
        __asm__ volatile("" : "+s"(voff));
        const float *lsel = (const float *)(ql + TILES);
        const float *dl = lsel + BLK;
        const bool pad_block = i == nb - 1 && (len & (BLK - 1)) != 0;
        if (pad_block) {
            // Q and dO rows past the end enter the transposed products: make them 0
            zero_tail_rows<D, NT>(ql, len - i * BLK, tid);
            zero_tail_rows<D, NT>(gl, len - i * BLK, tid);
            wait_vm_lgkm0<63>();
            workgroup_barrier();
        }
        if (i < lo_w || i > hi_w)
            continue;

        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = 0.0f;
            dp[r] = 0.0f;
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 qa = row_frag<D>(ql, col, 2 * ks + half);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ks], s, 0, 0, 0);
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 ga = row_frag<D>(gl, col, 2 * ks + half);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, row_frag<D>(ql + voff, col, 2 * ks + half), dp,
                                                         0, 0, 0);
        }
        const int di = i > j ? i - j : j - i;
        const bool need_mask = !kvalid || pad_block || (CAUSAL && i == j) ||
                               (p.window > 0 && di * BLK + BLK - 1 > p.window);
        // lse and D of this lane's 16 query rows, rows 8a + 4 half + (0..3),
        // four at a time: the empty asm stops the compiler from loading all
        // 32 values up front, which costs 24 registers
        float pv[16], ds[16];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 l4 = *(const f32x4 *)(lsel + 8 * a + 4 * half);
            const f32x4 d4 = *(const f32x4 *)(dl + 8 * a + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * a + e;
                const float pr = __builtin_amdgcn_exp2f(fmaf(s[r], c, -l4[e] * LOG2E));
                pv[r] = pr;
                ds[r] = pr * (dp[r] - d4[e]);
            }
            __asm__ volatile("" ::: "memory");
        }
        if (need_mask) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = i * BLK + acc_row(r, half);
                const int dist = qr > krow ? qr - krow : krow - qr;
                const bool keep = kvalid && qr < len && (!CAUSAL || krow <= qr) &&
                                  (p.window <= 0 || dist <= p.window);
                pv[r] = keep ? pv[r] : 0.0f;
                ds[r] = keep ? ds[r] : 0.0f;
            }
        }
        bf16x8 pb0, pb1, db0, db1;
        pack_b(pv, pb0, pb1);
        pack_b(ds, db0, db1);
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            bf16x8 a0, a1;
            tr_frags<D>(gl, m, tr_row, tr_col, a0, a1);
            dva[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pb0, dva[m], 0, 0, 0);
            dva[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pb1, dva[m], 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < NMT; ++m) {
            bf16x8 a0, a1;
            tr_frags<D>(ql, m, tr_row, tr_col, a0, a1);
            dka[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, db0, dka[m], 0, 0, 0);
            dka[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, db1, dka[m], 0, 0, 0);
        }
    }
    if (exists) {
        store_rowT<NMT>(dk_row, dka, p.scale, kvalid, half, !VARLEN || kvalid);
        store_rowT<NMT>(dv_row, dva, 1.0f, kvalid, half, !VARLEN || kvalid);
    }
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_bwd_v(const BwdLaunch &a, const BParams &p)
{
    constexpr int NS = 3;
    // dq also writes D (every row of every real block), which dkv reads
    hipLaunchKernelGGL((dq_kernel<D, NS, CAUSAL, VARLEN>), dim3(p.total), dim3(256), 0, a.stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    // dkv at d 128: a 2-stage ring, so that two workgroups (ring plus V tiles,
    // 64.5 KB each) share a CU's LDS; a third stage would need 80.75 KB
    constexpr int NSK = D == 128 ? 2 : NS;
    hipLaunchKernelGGL((dkv_kernel<D, NSK, CAUSAL, VARLEN>), dim3(p.total), dim3(256), 0, a.stream, p);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const BwdLaunch &a, const BParams &p)
{
    return a.cu_seqlens ? launch_bwd_v<D, CAUSAL, true>(a, p) : launch_bwd_v<D, CAUSAL, false>(a, p);
}

} // namespace

hipError_t launch_bwd_bf16(const BwdLaunch &a)
{
    BParams p;
    p.q = (const uint16_t *)a.q;
    p.k = (const uint16_t *)a.k;
    p.v = (const uint16_t *)a.v;
    p.o = (const uint16_t *)a.o;
    p.dout = (const uint16_t *)a.dout;
    p.lse = a.lse;
    p.seqlens = a.seqlens;
    p.cu = a.cu_seqlens;
    p.tokens = a.tokens;
    p.dq = (uint16_t *)a.dq;
    p.dk = (uint16_t *)a.dk;
    p.dv = (uint16_t *)a.dv;
    p.delta = a.delta;
    p.heads = a.heads;
    p.n = a.n;
    p.nblk = (a.n + BLK - 1) / BLK;
    p.ngroups = (p.nblk + 3) / 4;
    p.radius = a.radius;
    p.window = a.window;
    p.total = a.batch * a.heads * p.ngroups;
    p.c = a.scale * LOG2E;
    p.scale = a.scale;
    switch (a.head_dim) {
    case 64: return a.causal ? launch_bwd_d<64, true>(a, p) : launch_bwd_d<64, false>(a, p);
    case 128: return a.causal ? launch_bwd_d<128, true>(a, p) : launch_bwd_d<128, false>(a, p);
    default: return hipErrorInvalidValue;
    }
}

} // namespace bsl
