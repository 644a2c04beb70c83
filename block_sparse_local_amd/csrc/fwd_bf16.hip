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
//    it (up to 2R+1 of them).
//  * K and V blocks travel HBM -> LDS with direct-to-LDS buffer loads (no
//    registers; a scalar buffer resource per block, per-lane offsets fixed),
//    into a ring of NSTAGE buffers filled NSTAGE-1 blocks ahead of use; one
//    barrier per step both publishes the oldest block and frees the buffer the
//    previous step read.  16-byte chunks are XOR-swizzled per row so that the
//    MFMA operand reads below hit distinct LDS banks.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    in the 32x32 accumulator each lane then owns one query (column) and 16 of
//    the 32 keys, so the row maximum is 15 in-register max ops, plus one
//    exchange with the lane 32 away on the rare steps that move the reference
//    maximum; m, l and the rescale factor stay per lane.
//  * The output is also formed transposed, O^T += V^T P^T.  P^T is the MFMA B
//    operand straight from the score accumulator (rounded to bf16), with the key
//    order inside each 16-key step permuted to the accumulator's register order;
//    the matching V^T operand is read from the row-major V tile with the
//    transposing LDS read (ds_read_b64_tr_b16), four keys at a time.
//  * exp is the hardware 2^x with log2(e) folded into the score scale.  The
//    running maximum is only moved when a row's maximum grows by more than 2^8;
//    O / l is unchanged by the choice of reference point, and p stays <= 256.
//  * l is summed from the same bf16-rounded probabilities the PV product uses.
//  * Padded keys of the last block are masked by select (never by a multiply),
//    and their V rows are zeroed in LDS once the block has landed, so NaN
//    padding cannot leak.  A token window W (section 2, item 3, read as
//    |t - s| <= W) sweeps the ceil(W/32) blocks on either side and masks, by
//    the same select, only the blocks whose farthest pair lies beyond W.
//  * Workgroup ids are remapped so that each XCD (its own L2) works through a
//    contiguous run of query groups: neighbouring groups share K/V halo blocks.
//  * Vector memory instructions are what the texture addresser spends its time
//    on (about 34 of its cycles per 1 KB load), so the kernel issues as few as
//    it can: 16-byte loads and stores everywhere, O rows reassembled across
//    the lane pair that holds them before they are stored.
#include "cdna4.h"
#include "launch.h"

#include <math.h>

namespace bsl {
namespace {

// Design switches.  Each names one design choice of this kernel; the default
// is the shipped kernel, and every alternative computes the same result (same
// work, same masks, same arithmetic up to rounding), so that a build with one
// choice reverted can be timed and counted against the shipped one:
//   BSL_SWIZZLE       1: XOR-swizzle 16-byte chunks in LDS; 0: row-major tiles
//   BSL_XCD_REMAP     1: give each XCD a contiguous run of query groups;
//                     0: hardware order (groups dealt round robin to XCDs)
//   BSL_ROTATE        1: a full group visits key block j at step j mod P;
//                     0: every group sweeps its band from the left
//   BSL_RESCALE_SLACK move the reference maximum only when a row's maximum
//                     exceeds it by more than this (log2 units; 0: on any rise)
//   BSL_LAZY_EXCHANGE 1: exchange half-column maxima only on a move; 0: always
//   BSL_RING_BUFFER_LOADS 1: ring loads are buffer loads into LDS (a scalar
//                     resource per block, loop-invariant lane offsets);
//                     0: global loads into LDS with a 64-bit address per lane
//   BSL_WIDE_STORES   1: O rows reassembled across the lane pair and stored
//                     16 bytes at a time; 0: each lane stores its 8-byte halves
#ifndef BSL_SWIZZLE
#define BSL_SWIZZLE 1
#endif
#ifndef BSL_XCD_REMAP
#define BSL_XCD_REMAP 1
#endif
#ifndef BSL_ROTATE
#define BSL_ROTATE 1
#endif
#ifndef BSL_RESCALE_SLACK
#define BSL_RESCALE_SLACK 8.0f
#endif
#ifndef BSL_LAZY_EXCHANGE
#define BSL_LAZY_EXCHANGE 1
#endif
#ifndef BSL_RING_BUFFER_LOADS
#define BSL_RING_BUFFER_LOADS 1
#endif
#ifndef BSL_WIDE_STORES
#define BSL_WIDE_STORES 1
#endif

constexpr float RESCALE_SLACK = BSL_RESCALE_SLACK; // in log2 units

// Fourth word of a raw buffer resource on gfx9-family GPUs (32-bit data
// format, no swizzle, no index stride).
constexpr int BUFFER_WORD3 = 0x00020000;

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    const int32_t *seqlens; // padded layout: lengths (or nullptr)
    const int32_t *cu;      // packed layout: sequence start offsets, batch + 1 of them
    float *lse;
    int32_t *active;
    uint32_t *masks;
    // n: padded buffer length, or the longest sequence the grid covers (packed)
    int32_t heads, n, nblk, ngroups, radius, total;
    int32_t tokens; // packed layout: rows in the buffer
    int32_t window; // 0: the block band; >= 1: keys within this many tokens
    float c;        // scale * log2(e)
};

// Where sequence b's rows of head h live, and how many are real.  Padded layout
// [batch][heads][n][D]: rows D apart from (b heads + h) n D.  Packed layout
// [tokens][heads][D]: rows heads D apart from (cu[b] heads + h) D, lse
// [heads][tokens].  Offsets read from the device are clamped so that every row
// index below stays inside the buffer whatever they hold.
template <int D, bool VARLEN>
struct Seq {
    size_t base, lse_base;
    int len;
    __device__ __forceinline__ Seq(const Params &p, int b, int h, int bh)
    {
        if (VARLEN) {
            int s0 = p.cu[b], s1 = p.cu[b + 1];
            s0 = s0 < 0 ? 0 : (s0 > p.tokens ? p.tokens : s0);
            s1 = s1 < s0 ? s0 : (s1 > p.tokens ? p.tokens : s1);
            len = s1 - s0 > p.n ? p.n : s1 - s0;
            base = ((size_t)s0 * (size_t)p.heads + (size_t)h) * D;
            lse_base = (size_t)h * (size_t)p.tokens + (size_t)s0;
        } else {
            len = p.seqlens ? p.seqlens[b] : p.n;
            len = len < 0 ? 0 : (len > p.n ? p.n : len);
            base = (size_t)bh * (size_t)p.n * D;
            lse_base = (size_t)bh * (size_t)p.n;
        }
    }
};

// Workgroup order: each XCD's contiguous run of query groups (see
// xcd_contiguous), unless the design switch reverts to hardware order.
__device__ __forceinline__ int xcd_remap(int g, int total)
{
    return BSL_XCD_REMAP ? xcd_contiguous(g, total) : g;
}

// LDS tile geometry for head dim D: 32 rows of D bf16, row-major, CPR 16-byte
// chunks per row, chunk c of row r stored at chunk position c ^ swizzle(r).
template <int D>
struct Tile {
    static constexpr int CPR = D / 8;
    static constexpr int BYTES = BLK * D * 2;
    static constexpr int ROWS_PER_256B = 16 / CPR;
    // K is read as 32 rows x one logical chunk: spread 16 consecutive rows over
    // 16 distinct chunk positions of a 256-byte bank window.
    __device__ static __forceinline__ int k_swz(int r) { return BSL_SWIZZLE ? (r / ROWS_PER_256B) % CPR : 0; }
    // V is read 4 consecutive rows x 4 consecutive logical chunks at a time
    // (transposing reads): put the 4 rows in 4 different aligned 4-chunk sets.
    __device__ static __forceinline__ int v_swz(int r)
    {
        return BSL_SWIZZLE ? ((r / ROWS_PER_256B) & (CPR / 4 - 1)) << 2 : 0;
    }
};

template <int D, int MQ, int NSTAGE, bool CAUSAL, bool TRACE, bool VARLEN>
__global__ void __launch_bounds__(MQ * 64) fwd_bf16_kernel(Params p)
{
    using T = Tile<D>;
    static_assert(!(TRACE && VARLEN), "the trace describes the padded layout");
    // distance between consecutive rows of one head, in elements
    const size_t RS = VARLEN ? (size_t)p.heads * D : (size_t)D;
    constexpr int NT = MQ * 64;
    constexpr int NMT = D / 32;                 // 32-wide output tiles
    constexpr int NKS = D / 16;                 // 16-deep steps of the score contraction
    constexpr int STAGE = 2 * T::BYTES;         // K tile then V tile
    constexpr int SLOTS = STAGE / 16;           // 16-byte slots per stage
    static_assert(SLOTS % NT == 0 || NT % SLOTS == 0, "slots split evenly over waves");
    // direct-to-LDS loads per thread per block (waves past the last slot issue none)
    constexpr int LPT = SLOTS >= NT ? SLOTS / NT : 1;
    static_assert(T::BYTES % (64 * 16) == 0, "a wave's load covers only K or only V");
    static_assert(D % 32 == 0 && D <= 128, "head_dim must be 32, 64 or 128");
    static_assert(NSTAGE >= 2, "ring depth");

    __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 31, half = lane >> 5;

    const int g = xcd_remap((int)blockIdx.x, p.total);
    // Padded layout: a head's query groups are consecutive, so a run of groups
    // streams through one contiguous [n][D] slice.  Packed layout: a token's
    // heads sit side by side in memory.  With pieces of 128 bytes per head and
    // row (D 64 or less) the heads of one query group run consecutively, so a
    // run of groups reads whole token rows; with 256-byte pieces each piece is
    // already two full lines, and head-major order (as padded) keeps the
    // groups that share a head's halo blocks side by side, in the same L2 at
    // the same time.
    constexpr bool HEADS_FASTEST = VARLEN && D * 2 < 256;
    const int grp = HEADS_FASTEST ? (g / p.heads) % p.ngroups : g % p.ngroups;
    const int b = HEADS_FASTEST ? g / p.heads / p.ngroups : g / p.ngroups / p.heads;
    const int h = HEADS_FASTEST ? g % p.heads : (g / p.ngroups) % p.heads;
    const int bh = b * p.heads + h;
    const Seq<D, VARLEN> sq(p, b, h, bh);
    const int len = sq.len;
    const int nb = (len + BLK - 1) / BLK;
    const int R = p.radius, W = 2 * R + 1;
    const int i0 = grp * MQ;
    const int i = i0 + wave;
    // packed layout: rows past the sequence belong to the next one, so only the
    // sequence's own blocks exist; padded layout: every block of the buffer does
    // (blocks of padding get zero rows)
    const bool exists = i < (VARLEN ? nb : p.nblk);
    const bool trace_here = TRACE && h == 0;

    const size_t base = sq.base;
    const uint16_t *qg = p.q + base;
    const uint16_t *kg = p.k + base;
    const uint16_t *vg = p.v + base;
    uint16_t *og = p.o + base;
    const size_t trace_row = ((size_t)b * p.nblk + (size_t)i) * (size_t)W;

    // ------------------------------------------------ blocks of pure padding
    if (i0 >= nb) {
        if (!VARLEN && exists) {
            uint16_t *ob = og + (size_t)i * BLK * D;
            for (int c = lane; c < BLK * D / 8; c += 64)
                *(u32x4 *)(ob + (size_t)c * 8) = u32x4{0, 0, 0, 0};
            if (p.lse && half == 0)
                p.lse[sq.lse_base + (size_t)i * BLK + col] = -INFINITY;
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
    // Sweep order.  A full-width group visits key block j at step j mod P (P =
    // the width of a full group's band union), so the neighbouring groups that
    // share a halo block (on the same XCD, run at the same time) ask for it in
    // the same step and L2 serves all but the first request.  Softmax
    // accumulation does not depend on the order of the blocks.
    const int L = jhi - jlo + 1;
    const int P = CAUSAL ? MQ + R : MQ + 2 * R;
    const int rot = BSL_ROTATE && L == P ? (P - jlo % P) % P : 0;
    auto block_at = [&](int t) {
        const int x = t + rot;
        return jlo + (x >= L ? x - L : x);
    };

    // ------------------------------------------- K/V ring: direct-to-LDS
    // Slot s of a stage (16 bytes at stage + 16 s) holds K (s < SLOTS/2) or V;
    // within a tile, slot -> (row, chunk position), chunk position -> logical
    // chunk through the row's swizzle.  Load u of wave w fills slots
    // [u*NT + 64w, +64): 1 KB of LDS, 1 KB of contiguous global rows.  The
    // loads are buffer loads into LDS: a buffer resource (scalar registers)
    // based at the key block's first row, plus a loop-invariant per-lane byte
    // offset, so a step spends no vector ALU on addresses and the hardware
    // bounds-checks every access against the block.
    uint32_t loff[LPT];
#pragma unroll
    for (int u = 0; u < LPT; ++u) {
        const int s = u * NT + tid;
        const bool is_v = s >= SLOTS / 2;
        const int t = is_v ? s - SLOTS / 2 : s;
        const int r = t / T::CPR, cp = t % T::CPR;
        const int c = cp ^ (is_v ? T::v_swz(r) : T::k_swz(r));
        loff[u] = (uint32_t)r * (uint32_t)(RS * 2) + (uint32_t)c * 16u;
    }
    const int blk_bytes = (int)((size_t)BLK * RS * 2);
    auto issue = [&](int j, int stage) {
        const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(kg + (size_t)j * BLK * RS), (short)0, blk_bytes, BUFFER_WORD3);
        const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(vg + (size_t)j * BLK * RS), (short)0, blk_bytes, BUFFER_WORD3);
#pragma unroll
        for (int u = 0; u < LPT; ++u) {
            if (SLOTS < NT && u * NT + wave * 64 >= SLOTS)
                continue; // whole waves only: SLOTS is a multiple of 64
            const bool is_v = u * NT + wave * 64 >= SLOTS / 2; // uniform per wave
            uint32_t off = loff[u];
            if (VARLEN && (j + 1) * BLK > len) {
                // packed layout, the sequence's last block: rows past the end
                // repeat the last row (in bounds; masked below); the padded
                // buffer holds all 32 rows of every block
                const int t = (is_v ? u * NT + tid - SLOTS / 2 : u * NT + tid);
                const int r = t / T::CPR;
                const int last = len - 1 - j * BLK;
                if (r > last)
                    off -= (uint32_t)(r - last) * (uint32_t)(RS * 2);
            }
            uint8_t *dst = lds + stage * STAGE + (u * NT + wave * 64) * 16;
            if (BSL_RING_BUFFER_LOADS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(is_v ? vrs : krs, (lds_void *)dst, 16, off, 0,
                                                         0, 0);
            else
                __builtin_amdgcn_global_load_lds(
                    (const void *)((const uint8_t *)(is_v ? vg : kg) + (size_t)j * BLK * RS * 2 + off),
                    (lds_void *)dst, 16, 0, 0);
        }
    };

    // ----------------------------------------------------------- Q fragment
    // Every lane loads, so that no load sits in a branch: a lane without a
    // query of its own reads the sequence's first row (it exists: len >= 1
    // here), and zeroes it by select below, once the loads have landed.
    const int qrow = i * BLK + col;
    const bool qvalid = exists && qrow < len;
    const int qread = qvalid ? qrow : 0;
    bf16x8 qf[NKS];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
        qf[s] = as_bf16x8(*(const u32x4 *)(qg + (size_t)qread * RS + s * 16 + half * 8));

    // Start the ring before waiting on anything.  Every stage but the last is
    // filled, a sweep shorter than that repeating its last block into a stage
    // it never reads, so that the count of loads in flight is the same on
    // every path.
#pragma unroll
    for (int a = 0; a < NSTAGE - 1; ++a)
        issue(block_at(a < L ? a : L - 1), a);
    // Wait for the Q fragment here, with the ring's loads still in flight.  The
    // empty asm takes Q over as its own result, so the loop below uses no
    // register loaded outside it; otherwise the compiler drains every load in
    // flight, the whole ring included, before entering the loop.
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
        if (!qvalid)
            qf[s] = as_bf16x8(u32x4{0, 0, 0, 0});
        __asm__ volatile("" : "+v"(qf[s]));
    }

    f32x16 oacc[NMT];
#pragma unroll
    for (int m = 0; m < NMT; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            oacc[m][r] = 0.0f;
    // reference maximum (log2 units).  Finite, so that a block whose keys all
    // lie outside a row's token window (all scores -inf) gives exp2(-inf) = 0
    // rather than exp2(-inf + inf); the first real score replaces it with
    // alpha = exp2(-1e30 - m) = 0, as -inf would.
    float m_used = -1.0e30f;
    float lsum = 0.0f;        // this lane's share of the denominator

    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    // transposing-read coordinates of this lane inside its 16-lane group
    const int grp16 = lane >> 4, li = lane & 15;
    const int tr_row = 4 * half + (li >> 2);            // + 16 s (+ 8)
    const int tr_col = 16 * (grp16 & 1) + 4 * (li & 3); // + 32 m

    for (int t = 0; t < L; ++t) {
        const int j = block_at(t);
        const int stage = t % NSTAGE;
        // this wave's loads for step t are done once at most the loads of the
        // younger steps remain; then the barrier makes every wave's share visible
        // and frees the buffer read in the previous step
        if (!TRACE && t + NSTAGE - 2 < L)
            wait_vm_lgkm0<(NSTAGE - 2) * LPT>();
        else
            wait_vm_lgkm0<0>();
        workgroup_barrier();
        if (t + NSTAGE - 1 < L)
            issue(block_at(t + NSTAGE - 1), (t + NSTAGE - 1) % NSTAGE);
        const bool pad_block = j == nb - 1 && (len & (BLK - 1)) != 0;
        if (pad_block) {
            // the sequence ends inside this block: zero its V rows past the end
            // (whole rows, so the chunk swizzle does not matter), so that p = 0
            // never multiplies NaN or Inf padding; a later block loaded into
            // this buffer overwrites every row
            uint8_t *vz = lds + stage * STAGE + T::BYTES;
            const int r0 = len - j * BLK;
            for (int x = tid; x < (BLK - r0) * T::CPR; x += NT)
                *(u32x4 *)(vz + (r0 * T::CPR + x) * 16) = u32x4{0, 0, 0, 0};
            wait_vm_lgkm0<63>();
            workgroup_barrier();
        }

        if (j >= lo_w && j <= hi_w) {
            const uint8_t *kl = lds + stage * STAGE;
            const uint8_t *vl = kl + T::BYTES;

            // S^T = K_j Q_i^T  (rows: keys, columns: queries)
            f32x16 s;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c = (2 * ks + half) ^ T::k_swz(col);
                const bf16x8 a = as_bf16x8(*(const u32x4 *)(kl + col * D * 2 + c * 16));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s, 0, 0, 0);
            }

            // padding and causal masks: only the last real block and the
            // diagonal; a token window also cuts every block whose farthest
            // query-key pair, 32 |j - i| + 31 tokens apart, lies outside it
            const int dj = j > i ? j - i : i - j;
            const bool need_mask = pad_block || (CAUSAL && j == i) ||
                                   (p.window > 0 && dj * BLK + BLK - 1 > p.window);
            uint32_t part = 0;
            if (need_mask) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j * BLK + acc_row(r, half);
                    const int dist = qrow > key ? qrow - key : key - qrow;
                    const bool keep = key < len && (!CAUSAL || key <= qrow) &&
                                      (p.window <= 0 || dist <= p.window);
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

            // running maximum (log2 units), moved only when it grows a lot.  A
            // query's 32 scores sit in two lanes (l, l+32), 16 each; the column
            // maximum exceeds the bound exactly when one half's maximum does, so
            // the lanes test their own half and exchange only on the rare move
            // (the scale is positive, so scaling commutes with the maximum).
            float mx = s[0];
#pragma unroll
            for (int r = 1; r < 16; ++r)
                mx = fmaxf(mx, s[r]);
            const float mt_half = BSL_LAZY_EXCHANGE ? mx * p.c : fmaxf(mx, __shfl_xor(mx, 32)) * p.c;
            if (__ballot(mt_half > m_used + RESCALE_SLACK) != 0) {
                const float mt = BSL_LAZY_EXCHANGE ? fmaxf(mt_half, __shfl_xor(mt_half, 32)) : mt_half;
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
            const bf16x8 pb[2] = {as_bf16x8(u32x4{pk[0], pk[1], pk[2], pk[3]}),
                                  as_bf16x8(u32x4{pk[4], pk[5], pk[6], pk[7]})};

            // O^T += V_j^T P^T; the V^T operand comes from transposing reads
            const uint32_t vrow = (uint32_t)(size_t)(lds_u8 *)(vl + tr_row * D * 2 + (tr_col & 7) * 2);
            const int swz = T::v_swz(tr_row); // equal for rows +8, +16, +24
#pragma unroll
            for (int m = 0; m < NMT; ++m) {
                const int cp = (4 * m + (tr_col >> 3)) ^ swz;
                u32x2 r0, r1, r2, r3;
                tr_tile<D * 2>(vrow + cp * 16, r0, r1, r2, r3);
                const bf16x4 q0 = __builtin_bit_cast(bf16x4, r0), q1 = __builtin_bit_cast(bf16x4, r1);
                const bf16x4 q2 = __builtin_bit_cast(bf16x4, r2), q3 = __builtin_bit_cast(bf16x4, r3);
                const bf16x8 a0 = __builtin_shufflevector(q0, q1, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 a1 = __builtin_shufflevector(q2, q3, 0, 1, 2, 3, 4, 5, 6, 7);
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, pb[0], oacc[m], 0, 0, 0);
                oacc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, pb[1], oacc[m], 0, 0, 0);
            }
        }
    }

    // ------------------------------------------------------------- finalize
    const float lt = lsum + __shfl_xor(lsum, 32);
    if (!exists)
        return;
    // packed layout: a row past the sequence's end is the next sequence's
    if (VARLEN && !qvalid)
        return;
    const float inv = qvalid ? 1.0f / lt : 0.0f;
    uint16_t *orow = og + (size_t)qrow * RS;
    // Lanes l and l + 32 hold the two 4-element halves of each 8-element run
    // of the row; one exchange gives lane l the runs a = 0, 2 and lane l + 32
    // the runs a = 1, 3 whole, so the row leaves in 16-byte stores.
#pragma unroll
    for (int m = 0; m < NMT; ++m) {
        u32x2 pk4[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            f32x2 lo2 = {oacc[m][4 * a] * inv, oacc[m][4 * a + 1] * inv};
            f32x2 hi2 = {oacc[m][4 * a + 2] * inv, oacc[m][4 * a + 3] * inv};
            if (!qvalid) {
                lo2 = f32x2{0.0f, 0.0f};
                hi2 = f32x2{0.0f, 0.0f};
            }
            pk4[a] = u32x2{__builtin_bit_cast(uint32_t, __builtin_convertvector(lo2, bf16x2)),
                           __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2))};
        }
        if (!BSL_WIDE_STORES) {
#pragma unroll
            for (int a = 0; a < 4; ++a)
                *(u32x2 *)(orow + m * 32 + 8 * a + 4 * half) = pk4[a];
            continue;
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            // run a_mine = 2k + half is stored by this lane; the partner holds
            // its other half, and wants this lane's half of run 2k + 1 - half
            const u32x2 mine = half ? pk4[2 * k + 1] : pk4[2 * k];
            const u32x2 give = half ? pk4[2 * k] : pk4[2 * k + 1];
            u32x2 got;
            got[0] = (uint32_t)__shfl_xor((int)give[0], 32);
            got[1] = (uint32_t)__shfl_xor((int)give[1], 32);
            // d order inside the run: lane half 0 holds elements 0-3, half 1 holds 4-7
            const u32x4 run = half ? u32x4{got[0], got[1], mine[0], mine[1]}
                                   : u32x4{mine[0], mine[1], got[0], got[1]};
            *(u32x4 *)(orow + m * 32 + 8 * (2 * k + half)) = run;
        }
    }
    if (p.lse && half == 0)
        p.lse[sq.lse_base + (size_t)qrow] =
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

template <int D, int MQ, int NSTAGE, bool CAUSAL, bool TRACE, bool VARLEN>
hipError_t launch_t(const Launch &a, const Params &p)
{
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MQ, NSTAGE, CAUSAL, TRACE, VARLEN>), dim3(p.total),
                       dim3(MQ * 64), 0, a.stream, p);
    return hipGetLastError();
}

template <int D, int MQ, int NSTAGE>
hipError_t launch_d(const Launch &a, const Params &p)
{
    if (a.cu_seqlens)
        return a.causal ? launch_t<D, MQ, NSTAGE, true, false, true>(a, p)
                        : launch_t<D, MQ, NSTAGE, false, false, true>(a, p);
    const bool tr = a.active != nullptr;
    if (a.causal)
        return tr ? launch_t<D, MQ, NSTAGE, true, true, false>(a, p)
                  : launch_t<D, MQ, NSTAGE, true, false, false>(a, p);
    return tr ? launch_t<D, MQ, NSTAGE, false, true, false>(a, p)
              : launch_t<D, MQ, NSTAGE, false, false, false>(a, p);
}

} // namespace

// Query blocks (= waves) per workgroup and K/V ring depth: compile-time tuning
// knobs.  Measured on the d 128 / R 8 and d 64 / R 2 workloads: 4 and 3 are
// best.  Slower or no faster: 5, 6 or 8 query blocks per workgroup; rings of 2,
// 4 or 5 stages; a software-pipelined step (scores of block j+1 issued before
// the softmax of block j: 2 waves per SIMD instead of 3); all K operand reads
// issued ahead; the transposing V reads grouped 8 per wait; wave priority
// raised around the MFMA bursts; one wave per step issuing the whole ring
// refill; 5 waves per SIMD at d 64; and a persistent kernel with two query
// blocks per wave (1 wave per SIMD, whose MFMA, softmax and LDS waits then run
// back to back).
#ifndef BSL_BF16_MQ
#define BSL_BF16_MQ 4
#endif
#ifndef BSL_BF16_NSTAGE
#define BSL_BF16_NSTAGE 3
#endif

hipError_t launch_fwd_bf16(const Launch &a)
{
    constexpr int MQ = BSL_BF16_MQ;
    constexpr int NS = BSL_BF16_NSTAGE;
    Params p;
    p.q = (const uint16_t *)a.q;
    p.k = (const uint16_t *)a.k;
    p.v = (const uint16_t *)a.v;
    p.o = (uint16_t *)a.o;
    p.seqlens = a.seqlens;
    p.cu = a.cu_seqlens;
    p.lse = a.lse;
    p.active = a.active;
    p.masks = a.masks;
    p.heads = a.heads;
    p.n = a.n;
    p.tokens = a.tokens;
    p.nblk = (a.n + BLK - 1) / BLK;
    p.ngroups = (p.nblk + MQ - 1) / MQ;
    p.radius = a.radius;
    p.window = a.window;
    p.total = a.batch * a.heads * p.ngroups;
    p.c = a.scale * LOG2E;
    switch (a.head_dim) {
    case 32: return launch_d<32, MQ, NS>(a, p);
    case 64: return launch_d<64, MQ, NS>(a, p);
    case 128: return launch_d<128, MQ, NS>(a, p);
    default: return hipErrorInvalidValue;
    }
}

} // namespace bsl
